// Kernel launchers shared between the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "mxfp4spec.h"

namespace mxs {

// Compute units of the current device (cached per device).
int device_cus();

// Plain read of bytes (a multiple of 16) at buf, 16-byte aligned: the measured read ceiling.
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

// One product of a grouped verify GEMM (host-side view).
struct mxs_problem_view {
  const uint8_t* codes;
  const uint8_t* scales;
  const uint16_t* x;
  float* y;
  int64_t n;
  const float* gscale = nullptr;  // NVFP4 tensor scale (device), null for MX-FP4
};

hipError_t launch_verify_gemm_grouped(const mxs_problem_view* pv, int count, int64_t k, int64_t m,
                                      hipStream_t stream);

hipError_t launch_quantize(const float* w, int64_t n, int64_t k, uint8_t* codes, uint8_t* scales,
                           int32_t* flags, hipStream_t stream);

hipError_t launch_verify_gemm(const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t k,
                              const uint16_t* x, int64_t m, float* y, hipStream_t stream);

// Tiled codes (launch_tile_codes) and tiled scales (launch_tile_scales): the skinny kernel for
// m <= 32 with k % 512 == 0, else the dense kernel; k % 128 == 0 and k <= 2^23, checked by
// the caller. The grouped form takes up to 8 products per launch as the row layout's does.
hipError_t launch_verify_gemm_tiled(const uint8_t* tiled_codes, const uint8_t* tiled_scales, int64_t n, int64_t k,
                                    const uint16_t* x, int64_t m, float* y, hipStream_t stream);
hipError_t launch_verify_gemm_grouped_tiled(const mxs_problem_view* pv, int count, int64_t k, int64_t m,
                                            hipStream_t stream);

// Sampling transforms of spec_accept_sampled (validated by the caller).
struct SamplingParams {
  float temperature;      // > 0
  int32_t top_k;          // >= 0; 0 = off
  float top_p;            // (0, 1]; 1 = off
  const uint32_t* mask;   // [b][kd+1][ceil(v/32)] or null
};

hipError_t launch_nvfp4_quantize(const float* w, int64_t n, int64_t k, uint8_t* codes, uint8_t* scales,
                                 float* gscale, int32_t* flags, hipStream_t stream);

hipError_t launch_nvfp4_verify_gemm(const uint8_t* codes, const uint8_t* scales, const float* gscale,
                                    int64_t n, int64_t k, const uint16_t* x, int64_t m, float* y,
                                    hipStream_t stream);

// Several NVFP4 products with the same k (% 512 == 0) and m, each with its own tensor scale.
// The same with the codes in the tiled layout of launch_tile_codes (scales in the row layout).
hipError_t launch_nvfp4_verify_gemm_grouped_tiled(const mxs_problem_view* pv, int count, int64_t k, int64_t m,
                                                  hipStream_t stream);
hipError_t launch_nvfp4_verify_gemm_grouped(const mxs_problem_view* pv, int count, int64_t k, int64_t m,
                                            hipStream_t stream);

// MX-FP4 KV cache append: kv [t, heads, d] bf16 -> entries slots[i] of codes [capacity, heads, d/2]
// and scales [capacity, heads, d/32] (d % 32 == 0).
hipError_t launch_kv_append(const uint16_t* kv, int64_t t, int64_t heads, int64_t d, const int32_t* slots,
                            int64_t capacity, uint8_t* codes, uint8_t* scales, int32_t* flags, hipStream_t stream);

// MX activations (fmt MXS_ACT_FP8 or MXS_ACT_FP4) and the W4A8 / W4A4 product.
hipError_t launch_quantize_act(const uint16_t* x, int64_t m, int64_t k, int32_t fmt, uint8_t* codes,
                               uint8_t* scales, int32_t* flags, hipStream_t stream);

// tiled: codes in the layout of launch_tile_codes (16-row x 128-k tiles of 1 KiB) and
// scales in the layout of launch_tile_scales.
hipError_t launch_verify_gemm_act(const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t k,
                                  const uint8_t* act_codes, const uint8_t* act_scales, int32_t fmt,
                                  int64_t m, float* y, bool tiled, hipStream_t stream);

// Row-layout MX-FP4 codes [n, k/2] -> the tiled layout (k % 128 == 0; ceil(n/16)*16*k/2 bytes).
hipError_t launch_tile_codes(const uint8_t* codes, int64_t n, int64_t k, uint8_t* tiled, hipStream_t stream);

// Row-layout scales [n, k/32] -> 2 KiB per (128 rows, 512-k window) (k % 128 == 0;
// ceil(n/128) * ceil(k/512) * 2048 bytes).
hipError_t launch_tile_scales(const uint8_t* scales, int64_t n, int64_t k, uint8_t* tiled, hipStream_t stream);

size_t accept_workspace_bytes(int64_t b, int64_t kd, int64_t v, bool sampled);

// Top-k / top-p thresholds (order keys) of `rows` independent logit rows [rows, v] with masks
// [rows, ceil(v/32)] (sp.mask, or null): the selection spec_accept_sampled runs.
size_t sampling_thresholds_workspace_bytes(int64_t rows);
hipError_t launch_sampling_thresholds(const float* logits, int32_t rows, int32_t v, const SamplingParams& sp,
                                      uint32_t* out_thr, void* workspace, bool vec4, hipStream_t stream);

// Verification attention over the MX-FP4 KV cache (d = 128; rows = t * hq / hkv <= 64).
constexpr int kMaxAttnPositions = 64;
size_t kv_attention_workspace_bytes(int64_t b, int t, int hq, int hkv, int64_t max_len);
hipError_t launch_kv_attention(const uint16_t* q, const uint8_t* kc, const uint8_t* ks, const uint8_t* vc,
                               const uint8_t* vs, const int32_t* ctx, int32_t b, int32_t t, int32_t hq, int32_t hkv,
                               int64_t cap, int64_t max_len, const uint64_t* masks, float scale, float* out,
                               void* workspace, int32_t* flags, hipStream_t stream);

// Tree of draft tokens (spec_accept_tree): topology passed by value to the kernels.
constexpr int kMaxTreeNodes = 64;
constexpr int kMaxTreeChildren = 16;
struct TreeTopo {
  int n;       // draft nodes
  int depth;   // nodes on the longest root-to-leaf path
  int passes;  // residual passes: the largest child count + 1
  int8_t child[kMaxTreeNodes];    // nodes grouped by parent (the root's first), ascending
  int8_t off[kMaxTreeNodes + 2];  // children of row rho (0: root, i + 1: node i): child[off[rho] .. off[rho + 1])
};
size_t tree_workspace_bytes(int64_t b, const TreeTopo& topo, int64_t v);
hipError_t launch_spec_accept_tree(const float* target, const float* draft, const TreeTopo& topo,
                                   const int32_t* tokens, const float* uniforms, int32_t b, int32_t v,
                                   int32_t* out_tokens, int32_t* out_nodes, int32_t* out_num, void* workspace,
                                   int32_t* flags, bool vec4, hipStream_t stream);

// The built-in workspace of spec_accept_noalloc: a static device array of this many bytes
// (one per GPU, kept until the process ends). noalloc_scratch returns its device address
// on the current device, looked up once per device with hipGetSymbolAddress.
constexpr size_t kNoAllocScratchBytes = MXS_NOALLOC_SCRATCH_BYTES;
hipError_t noalloc_scratch(void** ptr);

// sp == nullptr: the plain laws (no transform kernels, the same code as without transforms).
hipError_t launch_spec_accept(const float* target, const float* draft, const int32_t* tokens,
                              const float* uniforms, int32_t b, int32_t kd, int32_t v,
                              int32_t* out_tokens, int32_t* out_num, void* workspace,
                              int32_t* flags, bool vec4, const SamplingParams* sp,
                              hipStream_t stream);

}  // namespace mxs
