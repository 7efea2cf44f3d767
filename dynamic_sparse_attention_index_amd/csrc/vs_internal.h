// Internal launch entry points shared between the kernel files and the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/vs_attn.h"

namespace vs {

// Device address of the debug build's bounds-violation counter on the current
// device (looked up once per device); null in the release build.
int32_t* debug_word();

// A device view of a [H, N, D] tensor as the kernels use it.
struct TView {
  const void* ptr;
  int64_t sh, sn;  // strides in elements
};

int launch_block_mask(const int32_t* vert_idx, const int32_t* vert_cnt, int64_t vert_stride,
                      const int32_t* slash_idx, const int32_t* slash_cnt, int64_t slash_stride,
                      int rank, int src, vs_mask* m, hipStream_t stream);

int launch_block_mask_ring(const int32_t* vert_idx, const int32_t* vert_cnt, int64_t vert_stride,
                           const int32_t* slash_idx, const int32_t* slash_cnt, int64_t slash_stride,
                           int rank, vs_mask* ms, int nsteps, hipStream_t stream);

int launch_attn_fwd(int dtype, int D, TView q, TView k, TView v, const vs_mask* m, float scale,
                    float* o, float* lse, int accumulate, hipStream_t stream);

int launch_attn_fwd_ring(int dtype, TView q, TView k, TView v, const vs_mask* ms, int nsteps, float scale, float* o,
                         float* lse, int accumulate, hipStream_t stream);

int launch_attn_fwd_packed(int dtype, TView q, TView k, TView v, const vs_mask* m, float scale, float* o,
                           float* lse, int accumulate, int32_t* status, hipStream_t stream);

int launch_merge(float* o_acc, float* lse_acc, const float* o_step, const float* lse_step,
                 int Hq, int64_t Nq, int D, hipStream_t stream);

int launch_convert_f16(const void* src, void* dst, int64_t n, int32_t* status, hipStream_t stream);

int launch_bwd_prep_f16(const float* o, const void* dout, void* dout16, int Hq, int64_t Nq, int D, float* delta,
                        int32_t* status, hipStream_t stream);

int launch_bwd_prep(const float* o, int dtype, TView dout, int Hq, int64_t Nq, int D, float* delta,
                    hipStream_t stream);

int launch_attn_bwd(int dtype, int D, TView q, TView k, TView v, TView dout, const float* lse,
                    const float* delta, const vs_mask* m, float scale, float* dq, float* dk, float* dv,
                    int parts, hipStream_t stream);

int launch_attn_bwd_ring(int dtype, TView q, TView k, TView v, TView dout, const float* lse, const float* delta,
                         const vs_mask* ms, int nsteps, float scale, float* dq, float* dk, float* dv, int parts,
                         hipStream_t stream);

size_t index_workspace_bytes(int Hq, int Hkv, int64_t n_global, int D, int last_q);

int launch_index_build(int dtype, int D, TView q_last, int Hq, int last_q, TView k, int Hkv,
                       const vs_layout& lay, float scale, float top_p, float* vert_score,
                       float* slash_score, int32_t* vert_idx, int32_t* vert_cnt, int32_t* slash_idx,
                       int32_t* slash_cnt, void* ws, size_t ws_bytes, hipStream_t stream);

int launch_index_rank_stats(int dtype, int D, TView q_last, int Hq, int last_q, TView k_local, int Hkv,
                            const vs_layout& lay, int rank, float scale, float* stats, void* ws, size_t ws_bytes,
                            hipStream_t stream);

int launch_index_rank_mass(int dtype, int D, TView q_last, int Hq, int last_q, TView k_local, int Hkv,
                           const vs_layout& lay, int rank, float scale, const float* all_stats, float* vert_score,
                           float* slash_score, void* ws, size_t ws_bytes, hipStream_t stream);

size_t select_workspace_bytes(int Hq, int64_t n_global);

size_t group_select_workspace_bytes(int Hkv, int64_t n_global);

int launch_index_select_group(const float* vert_score, const float* slash_score, int Hq, int Hkv, int64_t N,
                              float top_p, int32_t* vert_idx, int32_t* vert_cnt, int32_t* slash_idx,
                              int32_t* slash_cnt, void* ws, size_t ws_bytes, hipStream_t stream);

// budget: VS_BUDGET_TOP_P / VS_BUDGET_TOP_K / VS_BUDGET_JOINT_TOP_P (0 / 1 / 2)
int launch_index_select(const float* vert_score, const float* slash_score, int Hq, int64_t n_global, int budget,
                        float top_p, int k_vert, int k_slash, int32_t* vert_idx, int32_t* vert_cnt,
                        int32_t* slash_idx, int32_t* slash_cnt, void* ws, size_t ws_bytes, hipStream_t stream);

}  // namespace vs
