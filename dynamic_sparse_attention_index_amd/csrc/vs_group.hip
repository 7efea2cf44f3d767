// Index selected per kv head (grouped-query attention): the vertical and
// slash scores of the q heads that share a kv head are averaged, the top-p
// budget is applied once per kv head, and every q head of the group receives
// the group's lists. All q heads of a group then have the same active set, so
// two of them can share one workgroup and every K/V tile copy of the sparse
// forward. The per-q-head selection (one top-p per q head, as the review's
// index takes it) is the default path; this is its per-kv-head variant.
#include "vs_common.h"
#include "vs_internal.h"

namespace vs {

// out[g][i] = (sum over the R heads of group g, ascending, of in[h][i]) / R,
// for `rows` = Hkv rows of n entries. One thread per entry.
__global__ void group_mean_kernel(const float* in, float* out, int Hkv, int R, int64_t n) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (int64_t)Hkv * n) return;
  const int64_t g = t / n, i = t % n;
  float acc = 0.f;
  for (int r = 0; r < R; ++r) acc += in[(g * R + r) * n + i];
  out[t] = acc * (1.f / (float)R);
}

// Copy the group lists to every q head: idx rows of `stride` entries, of which
// the first cnt[g] are valid (the rest is copied too, and holds no meaning).
__global__ void replicate_lists_kernel(const int32_t* gidx, const int32_t* gcnt, int32_t* idx, int32_t* cnt,
                                       int Hq, int R, int64_t stride) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (int64_t)Hq * stride) return;
  const int64_t h = t / stride, i = t % stride;
  const int64_t g = h / R;
  if (i < gcnt[g]) idx[t] = gidx[g * stride + i];
  if (i == 0) cnt[h] = gcnt[g];
}

struct GroupWs {
  size_t vs, ss, vi, vc, si, sc, sel, total;
};
static size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }
static GroupWs group_ws(int Hkv, int64_t N) {
  const int64_t T = N / 64;
  GroupWs w;
  size_t o = 0;
  w.vs = o; o += up256((size_t)Hkv * N * 4);
  w.ss = o; o += up256((size_t)Hkv * T * 4);
  w.vi = o; o += up256((size_t)Hkv * N * 4);
  w.vc = o; o += up256((size_t)Hkv * 4);
  w.si = o; o += up256((size_t)Hkv * T * 4);
  w.sc = o; o += up256((size_t)Hkv * 4);
  w.sel = o; o += up256(select_workspace_bytes(Hkv, N));
  w.total = o;
  return w;
}

size_t group_select_workspace_bytes(int Hkv, int64_t n_global) { return group_ws(Hkv, n_global).total; }

int launch_index_select_group(const float* vert_score, const float* slash_score, int Hq, int Hkv, int64_t N,
                              float top_p, int32_t* vert_idx, int32_t* vert_cnt, int32_t* slash_idx,
                              int32_t* slash_cnt, void* ws, size_t ws_bytes, hipStream_t stream) {
  const GroupWs w = group_ws(Hkv, N);
  if (ws_bytes < w.total) return VS_ERR_WORKSPACE;
  char* b = (char*)ws;
  float* gv = (float*)(b + w.vs);
  float* gs = (float*)(b + w.ss);
  int32_t* gvi = (int32_t*)(b + w.vi);
  int32_t* gvc = (int32_t*)(b + w.vc);
  int32_t* gsi = (int32_t*)(b + w.si);
  int32_t* gsc = (int32_t*)(b + w.sc);
  const int R = Hq / Hkv;
  const int64_t T = N / 64;
  const int tpb = 256;
  hipLaunchKernelGGL(group_mean_kernel, dim3((unsigned)(((int64_t)Hkv * N + tpb - 1) / tpb)), dim3(tpb), 0, stream,
                     vert_score, gv, Hkv, R, N);
  hipLaunchKernelGGL(group_mean_kernel, dim3((unsigned)(((int64_t)Hkv * T + tpb - 1) / tpb)), dim3(tpb), 0, stream,
                     slash_score, gs, Hkv, R, T);
  if (hipGetLastError() != hipSuccess) return VS_ERR_HIP;
  int st = launch_index_select(gv, gs, Hkv, N, 0, top_p, 0, 0, gvi, gvc, gsi, gsc, b + w.sel, w.total - w.sel,
                               stream);
  if (st != VS_OK) return st;
  hipLaunchKernelGGL(replicate_lists_kernel, dim3((unsigned)(((int64_t)Hq * N + tpb - 1) / tpb)), dim3(tpb), 0,
                     stream, gvi, gvc, vert_idx, vert_cnt, Hq, R, N);
  hipLaunchKernelGGL(replicate_lists_kernel, dim3((unsigned)(((int64_t)Hq * T + tpb - 1) / tpb)), dim3(tpb), 0,
                     stream, gsi, gsc, slash_idx, slash_cnt, Hq, R, T);
  return hipGetLastError() == hipSuccess ? VS_OK : VS_ERR_HIP;
}

}  // namespace vs
