// C-ABI entry points of the MX-FP4 verification library: argument validation
// (before any HIP call), the gfx950 device check, and dispatch to the kernels.
#include <math.h>
#include <string.h>

#include <atomic>

#include "internal.hpp"
#include "mxfp4spec.h"

namespace {

constexpr int kMaxDevices = 64;
// Per-device cache of the architecture check: 0 unknown, 1 gfx950, 2 other.
std::atomic<int> g_arch_ok[kMaxDevices];

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

mxs_status check_device() {
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) return MXS_ERR_DEVICE;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MXS_ERR_DEVICE;
  if (dev < kMaxDevices) {
    const int cached = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (cached == 1) return MXS_OK;
    if (cached == 2) return MXS_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MXS_ERR_DEVICE;
  const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) g_arch_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? MXS_OK : MXS_ERR_DEVICE;
}

mxs_status launched(hipError_t e) { return e == hipSuccess ? MXS_OK : MXS_ERR_LAUNCH; }

// Topology of a draft tree from its parent array (host): false if malformed or too large.
bool make_topo(const int32_t* parent, int32_t n, mxs::TreeTopo& t) {
  if (n < 0 || n > mxs::kMaxTreeNodes || (n > 0 && !parent)) return false;
  int cnt[mxs::kMaxTreeNodes + 1] = {0};
  int depth[mxs::kMaxTreeNodes] = {0};
  t = mxs::TreeTopo{};
  t.n = n;
  for (int i = 0; i < n; ++i) {
    const int p = parent[i];
    if (p < -1 || p >= i) return false;
    ++cnt[p + 1];
    depth[i] = p < 0 ? 1 : depth[p] + 1;
    t.depth = depth[i] > t.depth ? depth[i] : t.depth;
  }
  int most = 0;
  t.off[0] = 0;
  for (int r = 0; r <= n; ++r) {
    t.off[r + 1] = (int8_t)(t.off[r] + cnt[r]);
    most = cnt[r] > most ? cnt[r] : most;
  }
  if (most > mxs::kMaxTreeChildren) return false;
  t.passes = most + 1;
  int pos[mxs::kMaxTreeNodes + 1];
  for (int r = 0; r <= n; ++r) pos[r] = t.off[r];
  for (int i = 0; i < n; ++i) t.child[pos[parent[i] + 1]++] = (int8_t)i;
  return true;
}

}  // namespace

extern "C" {

const char* mxs_status_string(int status) {
  switch (status) {
    case MXS_OK: return "MXS_OK";
    case MXS_ERR_NULL: return "MXS_ERR_NULL: a required pointer is NULL";
    case MXS_ERR_SHAPE: return "MXS_ERR_SHAPE: a size is out of range";
    case MXS_ERR_ALIGN: return "MXS_ERR_ALIGN: a pointer is misaligned";
    case MXS_ERR_WORKSPACE: return "MXS_ERR_WORKSPACE: workspace too small";
    case MXS_ERR_DEVICE: return "MXS_ERR_DEVICE: no usable gfx950 HIP device";
    case MXS_ERR_LAUNCH: return "MXS_ERR_LAUNCH: kernel launch failed";
    case MXS_ERR_VALUE: return "MXS_ERR_VALUE: an argument value is out of range";
    default: return "unknown mxs_status";
  }
}

int mxs_abi_version(void) { return MXS_ABI_VERSION; }

mxs_status mxfp4_quantize(const float* w, int64_t n, int64_t k, uint8_t* codes, uint8_t* scales,
                          int32_t* dev_flags, void* stream) {
  if (!w || !codes || !scales) return MXS_ERR_NULL;
  if (n < 1 || k < 32 || k % 32 != 0) return MXS_ERR_SHAPE;
  if (n > (int64_t(1) << 40) / k) return MXS_ERR_SHAPE;  // element count below 2^40
  if (!aligned(w, 16) || !aligned(codes, 16) || !aligned(dev_flags, 4)) return MXS_ERR_ALIGN;
  const mxs_status d = check_device();
  if (d != MXS_OK) return d;
  return launched(mxs::launch_quantize(w, n, k, codes, scales, dev_flags,
                                       static_cast<hipStream_t>(stream)));
}

mxs_status mxfp4_verify_gemm(const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t k,
                             const uint16_t* x, int64_t m, float* y, void* stream) {
  if (!codes || !scales || !x || !y) return MXS_ERR_NULL;
  if (n < 1 || k < 32 || k % 32 != 0 || m < 1 || m > 65536) return MXS_ERR_SHAPE;
  if (n > (int64_t(1) << 31) - 16 || k > (int64_t(1) << 30)) return MXS_ERR_SHAPE;
  if (!aligned(codes, 16) || !aligned(x, 16) || !aligned(y, 4)) return MXS_ERR_ALIGN;
  const mxs_status d = check_device();
  if (d != MXS_OK) return d;
  return launched(
      mxs::launch_verify_gemm(codes, scales, n, k, x, m, y, static_cast<hipStream_t>(stream)));
}

mxs_status mxfp4_verify_gemm_grouped(const mxs_gemm_problem* problems, int32_t count, int64_t k,
                                     int64_t m, void* stream) {
  if (!problems) return MXS_ERR_NULL;
  if (count < 1 || count > 65536 || k < 32 || k % 32 != 0 || k > (int64_t(1) << 30) || m < 1 ||
      m > 65536)
    return MXS_ERR_SHAPE;
  for (int32_t i = 0; i < count; ++i) {
    const mxs_gemm_problem& p = problems[i];
    if (!p.codes || !p.scales || !p.x || !p.y) return MXS_ERR_NULL;
    if (p.n < 1 || p.n > (int64_t(1) << 31) - 16) return MXS_ERR_SHAPE;
    if (!aligned(p.codes, 16) || !aligned(p.x, 16) || !aligned(p.y, 4)) return MXS_ERR_ALIGN;
  }
  const mxs_status d = check_device();
  if (d != MXS_OK) return d;
  constexpr int kBatch = 64;  // descriptors converted per host-side batch
  mxs::mxs_problem_view pv[kBatch];
  for (int32_t i0 = 0; i0 < count; i0 += kBatch) {
    const int cnt = count - i0 < kBatch ? count - i0 : kBatch;
    for (int j = 0; j < cnt; ++j) {
      const mxs_gemm_problem& p = problems[i0 + j];
      pv[j] = mxs::mxs_problem_view{p.codes, p.scales, p.x, p.y, p.n};
    }
    const mxs_status st =
        launched(mxs::launch_verify_gemm_grouped(pv, cnt, k, m, static_cast<hipStream_t>(stream)));
    if (st != MXS_OK) return st;
  }
  return MXS_OK;
}

mxs_status nvfp4_quantize(const float* w, int64_t n, int64_t k, uint8_t* codes, uint8_t* scales,
                          float* global_scale, int32_t* dev_flags, void* stream) {
  if (!w || !codes || !scales || !global_scale) return MXS_ERR_NULL;
  if (n < 1 || k < 16 || k % 16 != 0) return MXS_ERR_SHAPE;
  if (n > (int64_t(1) << 40) / k) return MXS_ERR_SHAPE;
  if (!aligned(w, 16) || !aligned(codes, 2) || !aligned(global_scale, 4) || !aligned(dev_flags, 4))
    return MXS_ERR_ALIGN;
  const mxs_status d = check_device();
  if (d != MXS_OK) return d;
  return launched(mxs::launch_nvfp4_quantize(w, n, k, codes, scales, global_scale, dev_flags,
                                             static_cast<hipStream_t>(stream)));
}

mxs_status nvfp4_verify_gemm(const uint8_t* codes, const uint8_t* scales, const float* global_scale,
                             int64_t n, int64_t k, const uint16_t* x, int64_t m, float* y,
                             void* stream) {
  if (!codes || !scales || !global_scale || !x || !y) return MXS_ERR_NULL;
  if (n < 1 || n > (int64_t(1) << 31) - 1 || k < 512 || k % 512 != 0 || k > (int64_t(1) << 24) ||
      m < 1 || m > 65536)
    return MXS_ERR_SHAPE;
  if (!aligned(codes, 16) || !aligned(scales, 16) || !aligned(global_scale, 4) || !aligned(x, 16) ||
      !aligned(y, 4))
    return MXS_ERR_ALIGN;
  const mxs_status d = check_device();
  if (d != MXS_OK) return d;
  return launched(mxs::launch_nvfp4_verify_gemm(codes, scales, global_scale, n, k, x, m, y,
                                                static_cast<hipStream_t>(stream)));
}

mxs_status nvfp4_verify_gemm_grouped(const mxs_nvfp4_problem* problems, int32_t count, int64_t k, int64_t m,
                                     void* stream) {
  if (!problems) return MXS_ERR_NULL;
  if (count < 1 || count > 65536 || k < 512 || k % 512 != 0 || k > (int64_t(1) << 24) || m < 1 || m > 65536)
    return MXS_ERR_SHAPE;
  for (int32_t i = 0; i < count; ++i) {
    const mxs_nvfp4_problem& p = problems[i];
    if (!p.codes || !p.scales || !p.global_scale || !p.x || !p.y) return MXS_ERR_NULL;
    if (p.n < 1 || p.n > (int64_t(1) << 31) - 1) return MXS_ERR_SHAPE;
    if (!aligned(p.codes, 16) || !aligned(p.scales, 16) || !aligned(p.global_scale, 4) || !aligned(p.x, 16) ||
        !aligned(p.y, 4))
      return MXS_ERR_ALIGN;
  }
  const mxs_status d = check_device();
  if (d != MXS_OK) return d;
  constexpr int kBatch = 64;  // descriptors converted per host-side batch
  mxs::mxs_problem_view pv[kBatch];
  for (int32_t i0 = 0; i0 < count; i0 += kBatch) {
    const int cnt = count - i0 < kBatch ? count - i0 : kBatch;
    for (int j = 0; j < cnt; ++j) {
      const mxs_nvfp4_problem& p = problems[i0 + j];
      pv[j] = mxs::mxs_problem_view{p.codes, p.scales, p.x, p.y, p.n, p.global_scale};
    }
    const mxs_status st =
        launched(mxs::launch_nvfp4_verify_gemm_grouped(pv, cnt, k, m, static_cast<hipStream_t>(stream)));
    if (st != MXS_OK) return st;
  }
  return MXS_OK;
}

mxs_status nvfp4_verify_gemm_grouped_tiled(const mxs_nvfp4_problem* problems, int32_t count, int64_t k, int64_t m,
                                           void* stream) {
  if (!problems) return MXS_ERR_NULL;
  if (count < 1 || count > 65536 || k < 512 || k % 512 != 0 || k > (int64_t(1) << 24) || m < 1 || m > 65536)
    return MXS_ERR_SHAPE;
  for (int32_t i = 0; i < count; ++i) {
    const mxs_nvfp4_problem& p = problems[i];
    if (!p.codes || !p.scales || !p.global_scale || !p.x || !p.y) return MXS_ERR_NULL;
    if (p.n < 1 || p.n > (int64_t(1) << 31) - 16) return MXS_ERR_SHAPE;
    if (!aligned(p.codes, 16) || !aligned(p.scales, 16) || !aligned(p.global_scale, 4) || !aligned(p.x, 16) ||
        !aligned(p.y, 4))
      return MXS_ERR_ALIGN;
  }
  const mxs_status d = check_device();
  if (d != MXS_OK) return d;
  constexpr int kBatch = 64;  // descriptors converted per host-side batch
  mxs::mxs_problem_view pv[kBatch];
  for (int32_t i0 = 0; i0 < count; i0 += kBatch) {
    const int cnt = count - i0 < kBatch ? count - i0 : kBatch;
    for (int j = 0; j < cnt; ++j) {
      const mxs_nvfp4_problem& p = problems[i0 + j];
      pv[j] = mxs::mxs_problem_view{p.codes, p.scales, p.x, p.y, p.n, p.global_scale};
    }
    const mxs_status st =
        launched(mxs::launch_nvfp4_verify_gemm_grouped_tiled(pv, cnt, k, m, static_cast<hipStream_t>(stream)));
    if (st != MXS_OK) return st;
  }
  return MXS_OK;
}

mxs_status mx_quantize_act(const uint16_t* x, int64_t m, int64_t k, int32_t fmt, uint8_t* codes,
                           uint8_t* scales, int32_t* dev_flags, void* stream) {
  if (!x || !codes || !scales) return MXS_ERR_NULL;
  if (fmt != MXS_ACT_FP8 && fmt != MXS_ACT_FP4) return MXS_ERR_VALUE;
  if (m < 1 || k < 32 || k % 32 != 0 || m > (int64_t(1) << 40) / k) return MXS_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(codes, fmt == MXS_ACT_FP8 ? 8 : 4) || !aligned(dev_flags, 4))
    return MXS_ERR_ALIGN;
  const mxs_status d = check_device();
  if (d != MXS_OK) return d;
  return launched(mxs::launch_quantize_act(x, m, k, fmt, codes, scales, dev_flags,
                                           static_cast<hipStream_t>(stream)));
}

mxs_status mx_verify_gemm_act(const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t k,
                              const uint8_t* act_codes, const uint8_t* act_scales, int32_t fmt, int64_t m,
                              float* y, void* stream) {
  if (!codes || !scales || !act_codes || !act_scales || !y) return MXS_ERR_NULL;
  if (fmt != MXS_ACT_FP8 && fmt != MXS_ACT_FP4) return MXS_ERR_VALUE;
  if (n < 1 || n > (int64_t(1) << 31) - 1 || k < 128 || k % 128 != 0 || k > (int64_t(1) << 24) ||
      m < 1 || m > 65536)
    return MXS_ERR_SHAPE;
  if (!aligned(codes, 16) || !aligned(act_codes, 16) || !aligned(scales, 4) || !aligned(act_scales, 4) ||
      !aligned(y, 4))
    return MXS_ERR_ALIGN;
  const mxs_status d = check_device();
  if (d != MXS_OK) return d;
  return launched(mxs::launch_verify_gemm_act(codes, scales, n, k, act_codes, act_scales, fmt, m, y, false,
                                              static_cast<hipStream_t>(stream)));
}

size_t mxfp4_tiled_bytes(int64_t n, int64_t k) {
  if (n < 1 || k < 128 || k % 128 != 0 || n > (int64_t(1) << 40) / k) return 0;
  return (size_t)((n + 15) / 16 * 16) * (size_t)(k / 2);
}

mxs_status mxfp4_tile_codes(const uint8_t* codes, int64_t n, int64_t k, uint8_t* tiled, void* stream) {
  if (!codes || !tiled) return MXS_ERR_NULL;
  if (n < 1 || k < 128 || k % 128 != 0 || n > (int64_t(1) << 40) / k) return MXS_ERR_SHAPE;
  if (!aligned(codes, 16) || !aligned(tiled, 16)) return MXS_ERR_ALIGN;
  const mxs_status d = check_device();
  if (d != MXS_OK) return d;
  return launched(mxs::launch_tile_codes(codes, n, k, tiled, static_cast<hipStream_t>(stream)));
}

size_t mxfp4_tiled_scale_bytes(int64_t n, int64_t k) {
  if (n < 1 || k < 128 || k % 128 != 0 || n > (int64_t(1) << 40) / k) return 0;
  return (size_t)((n + 127) / 128) * (size_t)((k + 511) / 512) * 2048u;
}

mxs_status mxfp4_tile_scales(const uint8_t* scales, int64_t n, int64_t k, uint8_t* tiled, void* stream) {
  if (!scales || !tiled) return MXS_ERR_NULL;
  if (n < 1 || k < 128 || k % 128 != 0 || n > (int64_t(1) << 40) / k) return MXS_ERR_SHAPE;
  if (!aligned(scales, 4) || !aligned(tiled, 16)) return MXS_ERR_ALIGN;
  const mxs_status d = check_device();
  if (d != MXS_OK) return d;
  return launched(mxs::launch_tile_scales(scales, n, k, tiled, static_cast<hipStream_t>(stream)));
}

mxs_status mx_verify_gemm_act_tiled(const uint8_t* tiled_codes, const uint8_t* tiled_scales, int64_t n, int64_t k,
                                    const uint8_t* act_codes, const uint8_t* act_scales, int32_t fmt, int64_t m,
                                    float* y, void* stream) {
  const uint8_t* scales = tiled_scales;
  if (!tiled_codes || !scales || !act_codes || !act_scales || !y) return MXS_ERR_NULL;
  if (fmt != MXS_ACT_FP8 && fmt != MXS_ACT_FP4) return MXS_ERR_VALUE;
  if (n < 1 || n > (int64_t(1) << 31) - 16 || k < 128 || k % 128 != 0 || k > (int64_t(1) << 24) || m < 1 ||
      m > 65536)
    return MXS_ERR_SHAPE;
  if (!aligned(tiled_codes, 16) || !aligned(act_codes, 16) || !aligned(scales, 16) || !aligned(act_scales, 4) ||
      !aligned(y, 4))
    return MXS_ERR_ALIGN;
  const mxs_status d = check_device();
  if (d != MXS_OK) return d;
  return launched(mxs::launch_verify_gemm_act(tiled_codes, scales, n, k, act_codes, act_scales, fmt, m, y, true,
                                              static_cast<hipStream_t>(stream)));
}

mxs_status mxfp4_verify_gemm_tiled(const uint8_t* tiled_codes, const uint8_t* tiled_scales, int64_t n, int64_t k,
                                   const uint16_t* x, int64_t m, float* y, void* stream) {
  if (!tiled_codes || !tiled_scales || !x || !y) return MXS_ERR_NULL;
  if (n < 1 || n > (int64_t(1) << 31) - 16 || k < 128 || k % 128 != 0 || k > (int64_t(1) << 23) || m < 1 ||
      m > 65536)
    return MXS_ERR_SHAPE;
  // the grid: 8 x ceil(n / 1024) row tiles x ceil(m / 80) position tiles of 512 threads
  if ((n + 1023) / 1024 * 8 * ((m + 79) / 80) > (int64_t)0xffffffffu / 512) return MXS_ERR_SHAPE;
  if (!aligned(tiled_codes, 16) || !aligned(tiled_scales, 16) || !aligned(x, 16) || !aligned(y, 4))
    return MXS_ERR_ALIGN;
  const mxs_status d = check_device();
  if (d != MXS_OK) return d;
  return launched(mxs::launch_verify_gemm_tiled(tiled_codes, tiled_scales, n, k, x, m, y,
                                                static_cast<hipStream_t>(stream)));
}

mxs_status mxfp4_verify_gemm_grouped_tiled(const mxs_gemm_problem* problems, int32_t count, int64_t k, int64_t m,
                                           void* stream) {
  if (!problems) return MXS_ERR_NULL;
  if (count < 1 || count > 65536 || k < 128 || k % 128 != 0 || k > (int64_t(1) << 23) || m < 1 || m > 65536)
    return MXS_ERR_SHAPE;
  for (int32_t i = 0; i < count; ++i) {
    const mxs_gemm_problem& p = problems[i];
    if (!p.codes || !p.scales || !p.x || !p.y) return MXS_ERR_NULL;
    if (p.n < 1 || p.n > (int64_t(1) << 31) - 16) return MXS_ERR_SHAPE;
    if ((p.n + 1023) / 1024 * 8 * ((m + 79) / 80) > (int64_t)0xffffffffu / 512) return MXS_ERR_SHAPE;
    if (!aligned(p.codes, 16) || !aligned(p.scales, 16) || !aligned(p.x, 16) || !aligned(p.y, 4))
      return MXS_ERR_ALIGN;
  }
  const mxs_status d = check_device();
  if (d != MXS_OK) return d;
  constexpr int kBatch = 64;  // descriptors converted per host-side batch
  mxs::mxs_problem_view pv[kBatch];
  for (int32_t i0 = 0; i0 < count; i0 += kBatch) {
    const int cnt = count - i0 < kBatch ? count - i0 : kBatch;
    for (int j = 0; j < cnt; ++j) {
      const mxs_gemm_problem& p = problems[i0 + j];
      pv[j] = mxs::mxs_problem_view{p.codes, p.scales, p.x, p.y, p.n};
    }
    const mxs_status st =
        launched(mxs::launch_verify_gemm_grouped_tiled(pv, cnt, k, m, static_cast<hipStream_t>(stream)));
    if (st != MXS_OK) return st;
  }
  return MXS_OK;
}

mxs_status mxfp4_kv_append(const uint16_t* kv, int64_t t, int64_t heads, int64_t d, const int32_t* slots,
                           int64_t capacity, uint8_t* codes, uint8_t* scales, int32_t* dev_flags, void* stream) {
  if (!kv || !slots || !codes || !scales) return MXS_ERR_NULL;
  if (t < 1 || heads < 1 || d < 32 || d % 32 != 0 || capacity < 1) return MXS_ERR_SHAPE;
  if (t > (int64_t(1) << 40) / (heads * d) || capacity > (int64_t(1) << 40) / (heads * d)) return MXS_ERR_SHAPE;
  if (!aligned(kv, 16) || !aligned(slots, 4) || !aligned(codes, 4) || !aligned(dev_flags, 4)) return MXS_ERR_ALIGN;
  const mxs_status dv = check_device();
  if (dv != MXS_OK) return dv;
  return launched(mxs::launch_kv_append(kv, t, heads, d, slots, capacity, codes, scales, dev_flags,
                                        static_cast<hipStream_t>(stream)));
}

size_t mxfp4_kv_attention_workspace_bytes(int32_t b, int32_t t, int32_t hq, int32_t hkv, int64_t max_len) {
  if (b < 1 || b > 65535 || t < 1 || t > mxs::kMaxAttnPositions || hkv < 1 || hq < hkv || hq % hkv != 0 ||
      t * (hq / hkv) > 64 || max_len < t || max_len > (int64_t(1) << 31))
    return 0;
  return mxs::kv_attention_workspace_bytes(b, t, hq, hkv, max_len);
}

mxs_status mxfp4_kv_attention(const uint16_t* q, const uint8_t* k_codes, const uint8_t* k_scales, const uint8_t* v_codes,
                              const uint8_t* v_scales, const int32_t* ctx_len, int32_t b, int32_t t, int32_t hq,
                              int32_t hkv, int32_t d, int64_t capacity, int64_t max_len, const uint64_t* masks,
                              float scale, float* out, void* workspace, size_t workspace_bytes, int32_t* dev_flags,
                              void* stream) {
  if (!q || !k_codes || !k_scales || !v_codes || !v_scales || !ctx_len || !masks || !out || !workspace)
    return MXS_ERR_NULL;
  if (b < 1 || b > 65535 || t < 1 || t > mxs::kMaxAttnPositions || hkv < 1 || hq < hkv || hq % hkv != 0 ||
      t * (hq / hkv) > 64 || d != 128 || max_len < t || max_len > capacity || capacity > (int64_t(1) << 31) ||
      (int64_t)b * capacity * hkv > (int64_t(1) << 34))
    return MXS_ERR_SHAPE;
  if (!(scale > 0.0f) || !(scale < INFINITY)) return MXS_ERR_VALUE;
  for (int i = 0; i < t; ++i)
    if (t < 64 && (masks[i] >> t)) return MXS_ERR_VALUE;  // a bit for a position past t (none at t = 64)
  if (!aligned(q, 16) || !aligned(k_codes, 16) || !aligned(v_codes, 16) || !aligned(ctx_len, 4) ||
      !aligned(out, 4) || !aligned(workspace, 16) || !aligned(dev_flags, 4))
    return MXS_ERR_ALIGN;
  if (workspace_bytes < mxs::kv_attention_workspace_bytes(b, t, hq, hkv, max_len)) return MXS_ERR_WORKSPACE;
  const mxs_status dv = check_device();
  if (dv != MXS_OK) return dv;
  return launched(mxs::launch_kv_attention(q, k_codes, k_scales, v_codes, v_scales, ctx_len, b, t, hq, hkv, capacity,
                                           max_len, masks, scale, out, workspace, dev_flags,
                                           static_cast<hipStream_t>(stream)));
}

mxs_status mxs_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink) return MXS_ERR_NULL;
  if (bytes < 16 || bytes % 16 != 0) return MXS_ERR_SHAPE;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return MXS_ERR_ALIGN;
  const mxs_status d = check_device();
  if (d != MXS_OK) return d;
  return launched(mxs::launch_stream_read(buf, bytes, sink, static_cast<hipStream_t>(stream)));
}

size_t spec_accept_tree_workspace_bytes(const int32_t* parent, int32_t nodes, int32_t b, int32_t v) {
  mxs::TreeTopo t;
  if (b < 1 || b > 65535 || v < 2 || v > (1 << 26) || !make_topo(parent, nodes, t)) return 0;
  return mxs::tree_workspace_bytes(b, t, v);
}

mxs_status spec_accept_tree(const float* target_logits, const float* draft_logits, const int32_t* parent,
                            int32_t nodes, const int32_t* draft_tokens, const float* uniforms, int32_t b, int32_t v,
                            int32_t* out_tokens, int32_t* out_nodes, int32_t* out_num_accepted, void* workspace,
                            size_t workspace_bytes, int32_t* dev_flags, void* stream) {
  if (!target_logits || !draft_logits || !uniforms || !out_tokens || !out_num_accepted || !workspace)
    return MXS_ERR_NULL;
  if (nodes > 0 && (!parent || !draft_tokens || !out_nodes)) return MXS_ERR_NULL;
  if (b < 1 || b > 65535 || v < 2 || v > (1 << 26) || nodes < 0 || nodes > mxs::kMaxTreeNodes) return MXS_ERR_SHAPE;
  mxs::TreeTopo t;
  if (!make_topo(parent, nodes, t)) return MXS_ERR_VALUE;
  if (!aligned(target_logits, 4) || !aligned(draft_logits, 4) || !aligned(draft_tokens, 4) ||
      !aligned(uniforms, 4) || !aligned(out_tokens, 4) || !aligned(out_nodes, 4) ||
      !aligned(out_num_accepted, 4) || !aligned(workspace, 16) || !aligned(dev_flags, 4))
    return MXS_ERR_ALIGN;
  if (workspace_bytes < mxs::tree_workspace_bytes(b, t, v)) return MXS_ERR_WORKSPACE;
  const mxs_status d = check_device();
  if (d != MXS_OK) return d;
  const bool vec4 = (v % 4 == 0) && aligned(target_logits, 16) && aligned(draft_logits, 16);
  return launched(mxs::launch_spec_accept_tree(target_logits, draft_logits, t, draft_tokens, uniforms, b, v,
                                               out_tokens, out_nodes, out_num_accepted, workspace, dev_flags, vec4,
                                               static_cast<hipStream_t>(stream)));
}

size_t spec_accept_workspace_bytes(int32_t b, int32_t kd, int32_t v) {
  if (b < 1 || b > 65535 || kd < 0 || kd > 32 || v < 2 || v > (1 << 26)) return 0;
  return mxs::accept_workspace_bytes(b, kd, v, false);
}

size_t spec_accept_sampled_workspace_bytes(int32_t b, int32_t kd, int32_t v) {
  if (b < 1 || b > 65535 || kd < 0 || kd > 32 || v < 2 || v > (1 << 26)) return 0;
  return mxs::accept_workspace_bytes(b, kd, v, true);
}

mxs_status spec_accept(const float* target_logits, const float* draft_logits,
                       const int32_t* draft_tokens, const float* uniforms, int32_t b, int32_t kd,
                       int32_t v, int32_t* out_tokens, int32_t* out_num_accepted, void* workspace,
                       size_t workspace_bytes, int32_t* dev_flags, void* stream) {
  if (!target_logits || !uniforms || !out_tokens || !out_num_accepted || !workspace)
    return MXS_ERR_NULL;
  if (kd > 0 && (!draft_logits || !draft_tokens)) return MXS_ERR_NULL;
  if (b < 1 || b > 65535 || kd < 0 || kd > 32 || v < 2 || v > (1 << 26)) return MXS_ERR_SHAPE;
  if (!aligned(target_logits, 4) || !aligned(draft_logits, 4) || !aligned(draft_tokens, 4) ||
      !aligned(uniforms, 4) || !aligned(out_tokens, 4) || !aligned(out_num_accepted, 4) ||
      !aligned(workspace, 16) || !aligned(dev_flags, 4))
    return MXS_ERR_ALIGN;
  if (workspace_bytes < mxs::accept_workspace_bytes(b, kd, v, false)) return MXS_ERR_WORKSPACE;
  const mxs_status d = check_device();
  if (d != MXS_OK) return d;
  const bool vec4 = (v % 4 == 0) && aligned(target_logits, 16) &&
                    (kd == 0 || aligned(draft_logits, 16));
  return launched(mxs::launch_spec_accept(target_logits, draft_logits, draft_tokens, uniforms, b,
                                          kd, v, out_tokens, out_num_accepted, workspace, dev_flags,
                                          vec4, nullptr, static_cast<hipStream_t>(stream)));
}

mxs_status spec_accept_noalloc(const float* target_logits, const float* draft_logits,
                               const int32_t* draft_tokens, const float* uniforms, int32_t b, int32_t kd,
                               int32_t v, int32_t* out_tokens, int32_t* out_num_accepted,
                               int32_t* dev_flags, void* stream) {
  if (!target_logits || !uniforms || !out_tokens || !out_num_accepted) return MXS_ERR_NULL;
  if (kd > 0 && (!draft_logits || !draft_tokens)) return MXS_ERR_NULL;
  if (b < 1 || b > 65535 || kd < 0 || kd > 32 || v < 2 || v > (1 << 26)) return MXS_ERR_SHAPE;
  if (!aligned(target_logits, 4) || !aligned(draft_logits, 4) || !aligned(draft_tokens, 4) ||
      !aligned(uniforms, 4) || !aligned(out_tokens, 4) || !aligned(out_num_accepted, 4) ||
      !aligned(dev_flags, 4))
    return MXS_ERR_ALIGN;
  if (mxs::accept_workspace_bytes(b, kd, v, false) > mxs::kNoAllocScratchBytes) return MXS_ERR_WORKSPACE;
  const mxs_status d = check_device();
  if (d != MXS_OK) return d;
  void* ws = nullptr;
  if (mxs::noalloc_scratch(&ws) != hipSuccess) return MXS_ERR_DEVICE;
  const bool vec4 = (v % 4 == 0) && aligned(target_logits, 16) &&
                    (kd == 0 || aligned(draft_logits, 16));
  return launched(mxs::launch_spec_accept(target_logits, draft_logits, draft_tokens, uniforms, b,
                                          kd, v, out_tokens, out_num_accepted, ws, dev_flags,
                                          vec4, nullptr, static_cast<hipStream_t>(stream)));
}

mxs_status spec_accept_sampled(const float* target_logits, const float* draft_logits,
                               const int32_t* draft_tokens, const float* uniforms, int32_t b,
                               int32_t kd, int32_t v, float temperature, int32_t top_k, float top_p,
                               const uint32_t* mask, int32_t* out_tokens, int32_t* out_num_accepted,
                               void* workspace, size_t workspace_bytes, int32_t* dev_flags,
                               void* stream) {
  if (!target_logits || !uniforms || !out_tokens || !out_num_accepted || !workspace)
    return MXS_ERR_NULL;
  if (kd > 0 && (!draft_logits || !draft_tokens)) return MXS_ERR_NULL;
  if (b < 1 || b > 65535 || kd < 0 || kd > 32 || v < 2 || v > (1 << 26)) return MXS_ERR_SHAPE;
  // NaN fails every comparison below
  if (!(temperature > 0.0f) || !(temperature < INFINITY) || top_k < 0 || !(top_p > 0.0f) ||
      !(top_p <= 1.0f))
    return MXS_ERR_VALUE;
  if (!aligned(target_logits, 4) || !aligned(draft_logits, 4) || !aligned(draft_tokens, 4) ||
      !aligned(uniforms, 4) || !aligned(out_tokens, 4) || !aligned(out_num_accepted, 4) ||
      !aligned(workspace, 16) || !aligned(dev_flags, 4) || !aligned(mask, 4))
    return MXS_ERR_ALIGN;
  if (workspace_bytes < mxs::accept_workspace_bytes(b, kd, v, true)) return MXS_ERR_WORKSPACE;
  const mxs_status d = check_device();
  if (d != MXS_OK) return d;
  const bool vec4 = (v % 4 == 0) && aligned(target_logits, 16) &&
                    (kd == 0 || aligned(draft_logits, 16));
  const mxs::SamplingParams sp{temperature, top_k, top_p, mask};
  return launched(mxs::launch_spec_accept(target_logits, draft_logits, draft_tokens, uniforms, b,
                                          kd, v, out_tokens, out_num_accepted, workspace, dev_flags,
                                          vec4, &sp, static_cast<hipStream_t>(stream)));
}

size_t spec_sampling_thresholds_workspace_bytes(int32_t rows, int32_t v) {
  if (rows < 1 || rows > (1 << 22) || v < 2 || v > (1 << 26)) return 0;
  return mxs::sampling_thresholds_workspace_bytes(rows);
}

mxs_status spec_sampling_thresholds(const float* logits, int32_t rows, int32_t v, float temperature,
                                    int32_t top_k, float top_p, const uint32_t* mask, uint32_t* out_thresholds,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  if (!logits || !out_thresholds || !workspace) return MXS_ERR_NULL;
  if (rows < 1 || rows > (1 << 22) || v < 2 || v > (1 << 26)) return MXS_ERR_SHAPE;
  if (!(temperature > 0.0f) || !(temperature < INFINITY) || top_k < 0 || !(top_p > 0.0f) ||
      !(top_p <= 1.0f))
    return MXS_ERR_VALUE;
  if (!aligned(logits, 4) || !aligned(out_thresholds, 4) || !aligned(workspace, 16) || !aligned(mask, 4))
    return MXS_ERR_ALIGN;
  if (workspace_bytes < mxs::sampling_thresholds_workspace_bytes(rows)) return MXS_ERR_WORKSPACE;
  const mxs_status d = check_device();
  if (d != MXS_OK) return d;
  const bool vec4 = (v % 4 == 0) && aligned(logits, 16);
  const mxs::SamplingParams sp{temperature, top_k, top_p, mask};
  return launched(mxs::launch_sampling_thresholds(logits, rows, v, sp, out_thresholds, workspace, vec4,
                                                  static_cast<hipStream_t>(stream)));
}

}  // extern "C"
