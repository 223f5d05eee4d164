// Host-side fuzz of the parameter packing (sampler_pack_host) and of the CPU
// oracle, built with -fsanitize=address,undefined by tests/test_sanitizers.py.
// Test infrastructure: it links the library's host code (sampler_abi.cpp)
// with no-op kernel launchers (no GPU is involved: sampler_pack_host makes no
// HIP call) and the oracle's C source.  Random batches mix valid rows with
// every kind of invalid value the ABI rejects; a sanitizer report aborts the
// process (non-zero exit).  The validation rules follow "SGLang 源码完全拆解(十)",
// section "后端分支" (fail fast on invalid parameters) and section
// "logit_bias 为什么用三元组构造" (CSR bias, the later duplicate wins).
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <random>
#include <vector>

#include "cd_sampler.h"
#include "kernels.h"

extern "C" {
#include "../../oracle/cd_oracle.h"
}

namespace cds {
hipError_t launch_transforms(const RowParams*, const int32_t*, const PenEntry*, const BiasEntry*,
                             float*, int64_t, int32_t, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_bitmask(void*, bool, int64_t, int32_t, int32_t, const int32_t*, int64_t,
                          const uint8_t*, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_fill_zero(void*, size_t, hipStream_t) { return hipSuccess; }
hipError_t static_workspace(void**, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_sample(const SampleArgs&, bool, bool, int, const KernelEvents*, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_outputs(const SampleArgs&, const OutputArgs&, bool, bool, const KernelEvents*,
                          hipStream_t) {
  return hipSuccess;
}
hipError_t launch_shard_pass(const ShardArgs&, bool, bool, hipStream_t) { return hipSuccess; }
hipError_t launch_shard_merge(const ShardArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_spec_accept(const SpecArgs&, hipStream_t) { return hipSuccess; }
}  // namespace cds

static int fail(const char* what, int it) {
  std::fprintf(stderr, "pack_fuzz: %s (iteration %d)\n", what, it);
  return 1;
}

int main(int argc, char** argv) {
  const int iters = argc > 1 ? std::atoi(argv[1]) : 3000;
  std::mt19937_64 rng(20261202);
  auto U = [&](double lo, double hi) { return std::uniform_real_distribution<double>(lo, hi)(rng); };
  auto I = [&](int64_t lo, int64_t hi) { return std::uniform_int_distribution<int64_t>(lo, hi)(rng); };
  const float kNaN = std::numeric_limits<float>::quiet_NaN();
  const float kInf = std::numeric_limits<float>::infinity();
  int ok_count = 0, rejected = 0;
  for (int it = 0; it < iters; ++it) {
    const int32_t B = (int32_t)I(1, 64);
    const int32_t V = (int32_t)(it % 17 == 0 ? I(1, 8) : I(1, 50000));
    std::vector<float> T(B), p(B), mp(B), rep(B), fr(B), pr(B);
    std::vector<int32_t> k(B);
    std::vector<uint64_t> seed(B), off(B);
    bool expect_bad = false;
    for (int32_t r = 0; r < B; ++r) {
      T[r] = I(0, 4) == 0 ? 0.0f : (float)U(1e-6, 2.0);
      k[r] = (int32_t)I(-2, V + 2);
      p[r] = I(0, 3) == 0 ? 1.0f : (float)U(1e-6, 1.0);
      mp[r] = I(0, 3) == 0 ? 0.0f : (float)U(0.0, 1.0);
      rep[r] = (float)U(0.5, 2.0);
      fr[r] = (float)U(-1.0, 1.0);
      pr[r] = (float)U(-1.0, 1.0);
      seed[r] = rng();
      off[r] = rng();
      // now and then one invalid value
      if (I(0, 40) == 0) {
        expect_bad = true;
        switch (I(0, 7)) {
          case 0: T[r] = -0.5f; break;
          case 1: T[r] = kNaN; break;
          case 2: p[r] = 0.0f; break;
          case 3: p[r] = 1.5f; break;
          case 4: mp[r] = kNaN; break;
          case 5: rep[r] = 0.0f; break;
          case 6: fr[r] = kInf; break;
          default: pr[r] = kNaN; break;
        }
      }
    }
    // history CSR: rows of 0 .. 6000 ids (some past the device-counted 4096)
    std::vector<int64_t> hp(B + 1, 0), bp(B + 1, 0);
    std::vector<int32_t> hid, bid;
    std::vector<float> bval;
    for (int32_t r = 0; r < B; ++r) {
      const int64_t n = I(0, 3) == 0 ? 0 : (I(0, 30) == 0 ? I(4090, 6000) : I(0, 600));
      for (int64_t i = 0; i < n; ++i) hid.push_back((int32_t)I(0, V - 1));
      hp[r + 1] = (int64_t)hid.size();
      const int64_t m = I(0, 40);
      for (int64_t i = 0; i < m; ++i) {
        bid.push_back((int32_t)I(0, std::min<int64_t>(V - 1, 20)));   // many duplicates
        bval.push_back(I(0, 20) == 0 ? -kInf : (float)U(-5.0, 5.0));
      }
      bp[r + 1] = (int64_t)bid.size();
    }
    if (!hid.empty() && I(0, 40) == 0) {
      hid[(size_t)I(0, (int64_t)hid.size() - 1)] = I(0, 1) ? V : -1;
      expect_bad = true;
    }
    if (!bid.empty() && I(0, 40) == 0) {
      bval[(size_t)I(0, (int64_t)bval.size() - 1)] = I(0, 1) ? kNaN : kInf;
      expect_bad = true;
    }
    sampler_host_params h;
    std::memset(&h, 0, sizeof h);
    h.B = B;
    h.V = V;
    h.temperature = T.data();
    h.top_k = k.data();
    h.top_p = p.data();
    h.min_p = mp.data();
    h.repetition_penalty = rep.data();
    h.frequency_penalty = fr.data();
    h.presence_penalty = pr.data();
    h.hist_indptr = hp.data();
    h.hist_ids = hid.empty() ? nullptr : hid.data();
    if (hid.empty()) h.hist_indptr = nullptr;
    h.bias_indptr = bid.empty() ? nullptr : bp.data();
    h.bias_ids = bid.empty() ? nullptr : bid.data();
    h.bias_vals = bid.empty() ? nullptr : bval.data();
    h.seed = seed.data();
    h.offset = I(0, 1) ? off.data() : nullptr;
    h.filter_order = (int32_t)I(0, 2);
    if (I(0, 60) == 0) {
      h.filter_order = I(0, 1) ? 3 : -1;
      expect_bad = true;
    }
    const size_t cap = sampler_params_bytes(B, (int64_t)hid.size(), (int64_t)bid.size());
    // an exact-size heap buffer: any write past the bound is an ASan report
    std::vector<unsigned char> buf(cap);
    sampler_batch out;
    const int rc = sampler_pack_host(&h, buf.data(), cap, &out);
    if (rc == SAMPLER_OK) {
      ++ok_count;
      if (expect_bad) return fail("an invalid batch was accepted", it);
      if (out.bytes > cap) return fail("packed size above the bound", it);
      if (out.B != B || out.V != V) return fail("shape not carried", it);
      if (out.n_sampled < 0 || out.n_sampled > B || out.n_hold > out.n_sampled)
        return fail("row counts out of range", it);
      // a too-small buffer must be refused, not overrun
      if (out.bytes > 1) {
        std::vector<unsigned char> small(out.bytes - 1);
        sampler_batch o2;
        if (sampler_pack_host(&h, small.data(), small.size(), &o2) != SAMPLER_ENOSPC)
          return fail("undersized buffer not refused", it);
      }
    } else {
      ++rejected;
      if (rc != SAMPLER_EINVAL && rc != SAMPLER_ERANGE) return fail("unexpected error code", it);
      if (!expect_bad) return fail("a valid batch was rejected", it);
    }
  }
  // the oracle on random rows: sizes 1 .. 3000, -inf / NaN / +inf / ties
  for (int it = 0; it < 400; ++it) {
    const int32_t V = (int32_t)I(1, 3000);
    std::vector<float> z(V);
    for (auto& v : z) v = (float)U(-6.0, 6.0);
    for (int32_t i = 0; i < V / 3; ++i) z[(size_t)I(0, V - 1)] = -kInf;
    if (I(0, 10) == 0) z[(size_t)I(0, V - 1)] = I(0, 1) ? kNaN : kInf;
    if (I(0, 5) == 0) for (auto& v : z) v = std::round(v);
    cdo_result res;
    std::vector<uint8_t> sets((size_t)V);
    cdo_sample_row(z.data(), V, I(0, 4) == 0 ? 0.0f : (float)U(1e-5, 3.0), (int32_t)I(-1, V + 1),
                   (float)U(1e-6, 1.0), (float)U(0.0, 1.0), rng(), rng(), &res,
                   it % 2 ? sets.data() : nullptr);
    if (res.status == 0 && (res.id < 0 || res.id >= V)) return fail("oracle id out of range", it);
  }
  std::printf("pack_fuzz: %d batches packed, %d rejected, oracle rows ok\n", ok_count, rejected);
  return 0;
}
