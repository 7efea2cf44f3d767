// The C ABI: host-side validation, workspace sizing and kernel launches.
// No device memory is allocated here; every buffer comes from the caller.
#include <string.h>

#include <mutex>

#include "vs_common.h"
#include "vs_internal.h"

using namespace vs;

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Float classification on the bit pattern: the library is built without NaN
// semantics, under which x != x and comparisons with NaN fold away.
uint32_t float_bits(float x) { uint32_t b; memcpy(&b, &x, 4); return b; }
bool is_nan(float x) { return (float_bits(x) & 0x7FFFFFFFu) > 0x7F800000u; }
bool finite_positive(float x) { const uint32_t b = float_bits(x); return b > 0u && b < 0x7F800000u; }

int elem_bytes(int dtype) { return dtype == VS_F32 ? 4 : 2; }

// Checks every property the kernels rely on for a [H, N, D] view.
int check_tensor(const vs_tensor& t, int H, int64_t N, int D) {
  if (!t.ptr) return VS_ERR_ARG;
  if (t.dtype != VS_F32 && t.dtype != VS_BF16 && t.dtype != VS_F16) return VS_ERR_ARG;
  if (t.H != H || t.N != N || t.D != D) return VS_ERR_ARG;
  if (t.stride_n < D || t.stride_h < 0) return VS_ERR_ARG;
  const int eb = elem_bytes(t.dtype);
  if (!aligned16(t.ptr) || (t.stride_n * eb) % 16 || (t.stride_h * eb) % 16) return VS_ERR_UNSUPPORTED;
  return VS_OK;
}

int check_layout(const vs_layout& lay) {
  if (lay.P < 1 || lay.n_global <= 0) return VS_ERR_ARG;
  if (lay.kind != VS_CONTIG && lay.kind != VS_STRIPED && lay.kind != VS_ZIGZAG && lay.kind != VS_STRIPED1)
    return VS_ERR_ARG;
  if (lay.kind == VS_STRIPED1 && lay.P > 32) return VS_ERR_UNSUPPORTED;
  const int64_t unit = (lay.kind == VS_ZIGZAG ? 128 : 64) * (int64_t)lay.P;
  if (lay.n_global % unit) return VS_ERR_UNSUPPORTED;
  if (lay.n_global / 64 > (int64_t)1 << 24) return VS_ERR_UNSUPPORTED;
  return VS_OK;
}

// index kernels: bf16 (D 64, 128) and f32 (D 64)
bool supported_dtype_dim(int dtype, int D) {
  return (dtype == VS_BF16 && (D == 64 || D == 128)) || (dtype == VS_F32 && D == 64);
}
// attention kernels: also fp16 at D = 128
bool supported_attn_dtype_dim(int dtype, int D) {
  return supported_dtype_dim(dtype, D) || (dtype == VS_F16 && D == 128);
}

TView view(const vs_tensor& t) { return TView{t.ptr, t.stride_h, t.stride_n}; }

struct MaskLayout {
  size_t off[12];
  size_t total;
};

MaskLayout mask_layout(int Hq, const vs_layout& lay, int64_t tile_cap) {
  const int64_t T = lay.n_global / 64, QB = T / lay.P, W = (T + 31) / 32;
  const size_t sizes[12] = {
      (size_t)(Hq * QB + 1) * 4,        // tile_ptr
      (size_t)tile_cap * 4,             // tile_col
      (size_t)(Hq * QB + 1) * 4,        // csc_ptr
      (size_t)tile_cap * 4,             // csc_row
      (size_t)(Hq * QB * 64) * 4,       // vloc
      (size_t)Hq * 4,                   // vloc_cnt
      (size_t)(Hq * (QB + 1)) * 4,      // vcum
      (size_t)(Hq * QB) * 4,            // vert_end
      (size_t)(Hq * W) * 4,             // slash_bits
      (size_t)(Hq * QB) * 8,            // n_active
      (size_t)4,                        // status
      0};
  MaskLayout L;
  size_t o = 0;
  for (int i = 0; i < 12; ++i) {
    L.off[i] = o;
    o += (sizes[i] + 255) & ~(size_t)255;
  }
  L.total = o;
  return L;
}

}  // namespace

extern "C" {

const char* vs_status_string(int s) {
  switch (s) {
    case VS_OK: return "ok";
    case VS_ERR_ARG: return "invalid argument";
    case VS_ERR_UNSUPPORTED: return "unsupported configuration";
    case VS_ERR_WORKSPACE: return "workspace or buffer too small";
    case VS_ERR_CAPACITY: return "tile list capacity exceeded";
    case VS_ERR_HIP: return "HIP runtime error";
    case VS_ERR_RANGE: return "value outside the range of the target type";
    default: return "unknown status";
  }
}

size_t vs_index_workspace_size(int Hq, int Hkv, int64_t n_global, int D, int last_q) {
  if (Hq <= 0 || Hkv <= 0 || n_global < 64) return 0;
  return index_workspace_bytes(Hq, Hkv, n_global, D, last_q);
}

int vs_index_build(vs_tensor q_last, vs_tensor k, vs_layout lay, float scale, float top_p,
                   float* vert_score, float* slash_score, int32_t* vert_idx, int32_t* vert_cnt,
                   int32_t* slash_idx, int32_t* slash_cnt, void* ws, size_t ws_bytes, void* stream) {
  int st;
  if ((st = check_layout(lay)) != VS_OK) return st;
  if (lay.kind == VS_STRIPED1 && lay.P > 1) return VS_ERR_UNSUPPORTED;   // keys in global order only
  const int Hq = q_last.H, Hkv = k.H, D = q_last.D, last_q = (int)q_last.N;
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv) return VS_ERR_ARG;
  if (Hq / Hkv > 8) return VS_ERR_UNSUPPORTED;
  if (last_q < 1 || last_q > 64) return VS_ERR_UNSUPPORTED;
  if ((st = check_tensor(q_last, Hq, last_q, D)) != VS_OK) return st;
  if ((st = check_tensor(k, Hkv, lay.n_global, D)) != VS_OK) return st;
  if (q_last.dtype != k.dtype || !supported_dtype_dim(k.dtype, D)) return VS_ERR_UNSUPPORTED;
  if (!vert_score || !slash_score || !vert_idx || !vert_cnt || !slash_idx || !slash_cnt || !ws)
    return VS_ERR_ARG;
  if (!finite_positive(scale) || is_nan(top_p)) return VS_ERR_ARG;
  if (ws_bytes < vs_index_workspace_size(Hq, Hkv, lay.n_global, D, last_q)) return VS_ERR_WORKSPACE;
  return launch_index_build(k.dtype, D, view(q_last), Hq, last_q, view(k), Hkv, lay, scale, top_p, vert_score,
                            slash_score, vert_idx, vert_cnt, slash_idx, slash_cnt, ws, ws_bytes,
                            (hipStream_t)stream);
}

// ---- the index build without a caller workspace ---------------------------
// Scratch of vs_index_build_noalloc: one copy per GPU the library runs on,
// held until the process ends. Host code never uses the array's name as an
// address (that is a host-side stand-in): each device's address is looked up
// once with hipGetSymbolAddress, with that device current, and kept.
static __device__ __align__(256) char scratch[VS_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
void* scratch_ptr[MAX_DEVICES] = {};

// This device's scratch address (looked up on its first use), or null.
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    scratch_ptr[dev] = p;
  }
  return scratch_ptr[dev];
}
}  // namespace

int vs_index_build_noalloc(vs_tensor q_last, vs_tensor k, vs_layout lay, float scale, float top_p,
                           float* vert_score, float* slash_score, int32_t* vert_idx, int32_t* vert_cnt,
                           int32_t* slash_idx, int32_t* slash_cnt, void* stream) {
  int st;
  if ((st = check_layout(lay)) != VS_OK) return st;
  const int Hq = q_last.H, Hkv = k.H, D = q_last.D, last_q = (int)q_last.N;
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv) return VS_ERR_ARG;
  // the size check comes first so that it needs no device
  if (vs_index_workspace_size(Hq, Hkv, lay.n_global, D, last_q) > (size_t)VS_NOALLOC_SCRATCH_BYTES)
    return VS_ERR_WORKSPACE;
  void* ws = device_scratch();
  if (!ws) return VS_ERR_HIP;
  return vs_index_build(q_last, k, lay, scale, top_p, vert_score, slash_score, vert_idx, vert_cnt, slash_idx,
                        slash_cnt, ws, (size_t)VS_NOALLOC_SCRATCH_BYTES, stream);
}

// ---- debug builds: bounds-violation counter ---------------------------------
// The bounds-checked build (VS_DEBUG_BOUNDS) counts, in one word per GPU, every
// mask value an attention kernel met outside the range its use allows (and
// replaced by an in-range one). Looked up per device like the scratch array.
}  // extern "C"

#ifdef VS_DEBUG_BOUNDS
static __device__ int32_t debug_count;
namespace {
int32_t* debug_ptr[MAX_DEVICES] = {};
}  // namespace
#endif

namespace vs {
int32_t* debug_word() {
#ifdef VS_DEBUG_BOUNDS
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!debug_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(debug_count)) != hipSuccess || !p) return nullptr;
    debug_ptr[dev] = (int32_t*)p;
  }
  return debug_ptr[dev];
#else
  return nullptr;
#endif
}
}  // namespace vs

extern "C" {

int vs_debug_bounds_enabled(void) {
#ifdef VS_DEBUG_BOUNDS
  return 1;
#else
  return 0;
#endif
}

int vs_debug_bounds_count(int32_t* count, int reset, void* stream) {
  if (!count || (reset != 0 && reset != 1)) return VS_ERR_ARG;
  *count = 0;
#ifdef VS_DEBUG_BOUNDS
  int32_t* w = debug_word();
  if (!w) return VS_ERR_HIP;
  hipStream_t s = (hipStream_t)stream;
  if (hipMemcpyAsync(count, w, sizeof(int32_t), hipMemcpyDeviceToHost, s) != hipSuccess) return VS_ERR_HIP;
  if (reset && hipMemsetAsync(w, 0, sizeof(int32_t), s) != hipSuccess) return VS_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return VS_ERR_HIP;
#else
  (void)stream;
#endif
  return VS_OK;
}

// Checks shared by the per-rank index calls; on success sets the dims.
static int check_rank_index(vs_tensor q_last, vs_tensor k_local, vs_layout lay, int rank, float scale, void* ws,
                            size_t ws_bytes, int* Hq, int* Hkv, int* D, int* last_q) {
  int st;
  if ((st = check_layout(lay)) != VS_OK) return st;
  if (lay.kind == VS_STRIPED1 && lay.P > 1) return VS_ERR_UNSUPPORTED;   // per-rank tiles span P blocks
  if (rank < 0 || rank >= lay.P) return VS_ERR_ARG;
  *Hq = q_last.H; *Hkv = k_local.H; *D = q_last.D; *last_q = (int)q_last.N;
  if (*Hq <= 0 || *Hkv <= 0 || *Hq % *Hkv) return VS_ERR_ARG;
  if (*Hq / *Hkv > 8) return VS_ERR_UNSUPPORTED;
  if (*last_q < 1 || *last_q > 64) return VS_ERR_UNSUPPORTED;
  if ((st = check_tensor(q_last, *Hq, *last_q, *D)) != VS_OK) return st;
  if ((st = check_tensor(k_local, *Hkv, lay.n_global / lay.P, *D)) != VS_OK) return st;
  if (q_last.dtype != k_local.dtype || !supported_dtype_dim(k_local.dtype, *D)) return VS_ERR_UNSUPPORTED;
  if (!ws || !finite_positive(scale)) return VS_ERR_ARG;
  if (ws_bytes < vs_index_workspace_size(*Hq, *Hkv, lay.n_global, *D, *last_q)) return VS_ERR_WORKSPACE;
  return VS_OK;
}

int vs_index_rank_stats(vs_tensor q_last, vs_tensor k_local, vs_layout lay, int rank, float scale,
                        float* stats, void* ws, size_t ws_bytes, void* stream) {
  int Hq, Hkv, D, last_q, st;
  if ((st = check_rank_index(q_last, k_local, lay, rank, scale, ws, ws_bytes, &Hq, &Hkv, &D, &last_q)) != VS_OK)
    return st;
  if (!stats) return VS_ERR_ARG;
  return launch_index_rank_stats(k_local.dtype, D, view(q_last), Hq, last_q, view(k_local), Hkv, lay, rank, scale,
                                 stats, ws, ws_bytes, (hipStream_t)stream);
}

int vs_index_rank_mass(vs_tensor q_last, vs_tensor k_local, vs_layout lay, int rank, float scale,
                       const float* all_stats, float* vert_score, float* slash_score,
                       void* ws, size_t ws_bytes, void* stream) {
  int Hq, Hkv, D, last_q, st;
  if ((st = check_rank_index(q_last, k_local, lay, rank, scale, ws, ws_bytes, &Hq, &Hkv, &D, &last_q)) != VS_OK)
    return st;
  if (!all_stats || !vert_score || !slash_score) return VS_ERR_ARG;
  return launch_index_rank_mass(k_local.dtype, D, view(q_last), Hq, last_q, view(k_local), Hkv, lay, rank, scale,
                                all_stats, vert_score, slash_score, ws, ws_bytes, (hipStream_t)stream);
}

size_t vs_index_select_workspace_size(int Hq, int64_t n_global) {
  if (Hq <= 0 || n_global <= 0) return 0;
  return select_workspace_bytes(Hq, n_global);
}

int vs_index_select_budget(const float* vert_score, const float* slash_score, int Hq, int64_t n_global, int budget,
                           float top_p, int k_vert, int k_slash, int32_t* vert_idx, int32_t* vert_cnt,
                           int32_t* slash_idx, int32_t* slash_cnt, void* ws, size_t ws_bytes, void* stream) {
  if (!vert_score || !slash_score || !vert_idx || !vert_cnt || !slash_idx || !slash_cnt || Hq <= 0 || !ws)
    return VS_ERR_ARG;
  if (budget != VS_BUDGET_TOP_P && budget != VS_BUDGET_TOP_K && budget != VS_BUDGET_JOINT_TOP_P) return VS_ERR_ARG;
  if (is_nan(top_p) || n_global <= 0) return VS_ERR_ARG;
  if (n_global % 64 || n_global > ((int64_t)1 << 30)) return VS_ERR_UNSUPPORTED;
  if (ws_bytes < select_workspace_bytes(Hq, n_global)) return VS_ERR_WORKSPACE;
  return launch_index_select(vert_score, slash_score, Hq, n_global, budget, top_p, k_vert, k_slash, vert_idx,
                             vert_cnt, slash_idx, slash_cnt, ws, ws_bytes, (hipStream_t)stream);
}

int vs_index_select(const float* vert_score, const float* slash_score, int Hq, int64_t n_global, float top_p,
                    int32_t* vert_idx, int32_t* vert_cnt, int32_t* slash_idx, int32_t* slash_cnt,
                    void* ws, size_t ws_bytes, void* stream) {
  return vs_index_select_budget(vert_score, slash_score, Hq, n_global, VS_BUDGET_TOP_P, top_p, 0, 0, vert_idx,
                                vert_cnt, slash_idx, slash_cnt, ws, ws_bytes, stream);
}

size_t vs_index_select_group_workspace_size(int Hq, int Hkv, int64_t n_global) {
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv || n_global <= 0 || n_global % 64) return 0;
  return group_select_workspace_bytes(Hkv, n_global);
}

int vs_index_select_group(const float* vert_score, const float* slash_score, int Hq, int Hkv, int64_t n_global,
                          float top_p, int32_t* vert_idx, int32_t* vert_cnt, int32_t* slash_idx, int32_t* slash_cnt,
                          void* ws, size_t ws_bytes, void* stream) {
  if (!vert_score || !slash_score || !vert_idx || !vert_cnt || !slash_idx || !slash_cnt || !ws) return VS_ERR_ARG;
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv || is_nan(top_p) || n_global <= 0) return VS_ERR_ARG;
  if (n_global % 64 || n_global > ((int64_t)1 << 30)) return VS_ERR_UNSUPPORTED;
  if (ws_bytes < group_select_workspace_bytes(Hkv, n_global)) return VS_ERR_WORKSPACE;
  return launch_index_select_group(vert_score, slash_score, Hq, Hkv, n_global, top_p, vert_idx, vert_cnt, slash_idx,
                                   slash_cnt, ws, ws_bytes, (hipStream_t)stream);
}

size_t vs_mask_bytes(int Hq, int Hkv, vs_layout lay, int64_t tile_cap) {
  if (Hq <= 0 || Hkv <= 0 || tile_cap < 0 || check_layout(lay) != VS_OK) return 0;
  return mask_layout(Hq, lay, tile_cap).total;
}

int vs_mask_init(vs_mask* m, void* buf, size_t bytes, int Hq, int Hkv, vs_layout lay, int64_t tile_cap) {
  int st;
  if (!m || !buf) return VS_ERR_ARG;
  if ((st = check_layout(lay)) != VS_OK) return st;
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv || tile_cap < 0 || tile_cap > 0x7FFFFFFF) return VS_ERR_ARG;
  if (!aligned16(buf)) return VS_ERR_UNSUPPORTED;
  const MaskLayout L = mask_layout(Hq, lay, tile_cap);
  if (bytes < L.total) return VS_ERR_WORKSPACE;
  memset(m, 0, sizeof(*m));
  char* b = (char*)buf;
  m->Hq = Hq;
  m->Hkv = Hkv;
  m->T = (int32_t)(lay.n_global / 64);
  m->QB = m->KB = m->T / lay.P;
  m->W = (m->T + 31) / 32;
  m->lay = lay;
  m->tile_cap = tile_cap;
  m->rank = m->src = -1;
  m->tile_ptr = (int32_t*)(b + L.off[0]);
  m->tile_col = (int32_t*)(b + L.off[1]);
  m->csc_ptr = (int32_t*)(b + L.off[2]);
  m->csc_row = (int32_t*)(b + L.off[3]);
  m->vloc = (int32_t*)(b + L.off[4]);
  m->vloc_cnt = (int32_t*)(b + L.off[5]);
  m->vcum = (int32_t*)(b + L.off[6]);
  m->vert_end = (int32_t*)(b + L.off[7]);
  m->slash_bits = (uint32_t*)(b + L.off[8]);
  m->n_active = (int64_t*)(b + L.off[9]);
  m->status = (int32_t*)(b + L.off[10]);
  return VS_OK;
}

int vs_block_mask(const int32_t* vert_idx, const int32_t* vert_cnt, int64_t vert_stride,
                  const int32_t* slash_idx, const int32_t* slash_cnt, int64_t slash_stride,
                  int rank, int step, vs_mask* m, void* stream) {
  if (!m || !m->tile_ptr || !vert_idx || !vert_cnt || !slash_idx || !slash_cnt) return VS_ERR_ARG;
  if (check_layout(m->lay) != VS_OK) return VS_ERR_ARG;
  const int P = m->lay.P;
  if (rank < 0 || rank >= P || step < 0 || step >= P) return VS_ERR_ARG;
  if (vert_stride < 0 || slash_stride < 0) return VS_ERR_ARG;
  const int src = ((rank - step) % P + P) % P;
  m->rank = rank;
  m->src = src;
  return launch_block_mask(vert_idx, vert_cnt, vert_stride, slash_idx, slash_cnt, slash_stride, rank, src, m,
                           (hipStream_t)stream);
}

int vs_block_mask_ring(const int32_t* vert_idx, const int32_t* vert_cnt, int64_t vert_stride,
                       const int32_t* slash_idx, const int32_t* slash_cnt, int64_t slash_stride,
                       int rank, vs_mask* masks, int nsteps, void* stream) {
  if (!masks || nsteps < 1 || !vert_idx || !vert_cnt || !slash_idx || !slash_cnt) return VS_ERR_ARG;
  if (vert_stride < 0 || slash_stride < 0) return VS_ERR_ARG;
  const vs_mask& m = masks[0];
  if (check_layout(m.lay) != VS_OK) return VS_ERR_ARG;
  const int P = m.lay.P;
  if (rank < 0 || rank >= P || nsteps > P) return VS_ERR_ARG;
  for (int s = 0; s < nsteps; ++s) {
    const vs_mask& x = masks[s];
    if (!x.tile_ptr || !x.tile_col || !x.csc_ptr || !x.csc_row || !x.vloc || !x.vloc_cnt || !x.vcum ||
        !x.vert_end || !x.slash_bits || !x.n_active || !x.status)
      return VS_ERR_ARG;
    if (x.Hq != m.Hq || x.Hkv != m.Hkv || x.QB != m.QB || x.KB != m.KB || x.T != m.T || x.W != m.W ||
        x.lay.kind != m.lay.kind || x.lay.P != P || x.lay.n_global != m.lay.n_global || x.tile_cap != m.tile_cap)
      return VS_ERR_ARG;
  }
  return launch_block_mask_ring(vert_idx, vert_cnt, vert_stride, slash_idx, slash_cnt, slash_stride, rank, masks,
                                nsteps, (hipStream_t)stream);
}

static int check_attn(const vs_tensor& q, const vs_tensor& k, const vs_tensor& v, const vs_mask* m) {
  int st;
  if (!m || !m->tile_ptr || m->rank < 0) return VS_ERR_ARG;
  const int D = q.D;
  const int64_t Nq = (int64_t)m->QB * 64, Nk = (int64_t)m->KB * 64;
  if ((st = check_tensor(q, m->Hq, Nq, D)) != VS_OK) return st;
  if ((st = check_tensor(k, m->Hkv, Nk, D)) != VS_OK) return st;
  if ((st = check_tensor(v, m->Hkv, Nk, D)) != VS_OK) return st;
  if (q.dtype != k.dtype || q.dtype != v.dtype) return VS_ERR_ARG;
  if (!supported_attn_dtype_dim(q.dtype, D)) return VS_ERR_UNSUPPORTED;
  // one-position stripes: the per-entry path of the head-dim-128 kernels
  if (m->lay.kind == VS_STRIPED1 && (D != 128 || q.dtype == VS_F32)) return VS_ERR_UNSUPPORTED;
  return VS_OK;
}

int vs_attn_fwd(vs_tensor q, vs_tensor k, vs_tensor v, const vs_mask* m, float scale, float* o, float* lse,
                int accumulate, void* stream) {
  int st;
  if ((st = check_attn(q, k, v, m)) != VS_OK) return st;
  if (!o || !lse || !aligned16(o)) return VS_ERR_ARG;
  if (accumulate != 0 && accumulate != 1) return VS_ERR_ARG;
  if (!finite_positive(scale)) return VS_ERR_ARG;
  return launch_attn_fwd(q.dtype, q.D, view(q), view(k), view(v), m, scale, o, lse, accumulate,
                         (hipStream_t)stream);
}

int vs_attn_fwd_packed(vs_tensor q, vs_tensor k, vs_tensor v, const vs_mask* m, float scale, float* o, float* lse,
                       int accumulate, int32_t* status, void* stream) {
  int st;
  if ((st = check_attn(q, k, v, m)) != VS_OK) return st;
  if (!o || !lse || !status || !aligned16(o)) return VS_ERR_ARG;
  if (accumulate != 0 && accumulate != 1) return VS_ERR_ARG;
  if (!finite_positive(scale)) return VS_ERR_ARG;
  if ((q.dtype != VS_BF16 && q.dtype != VS_F16) || q.D != 128 || (m->Hq / m->Hkv) % 2) return VS_ERR_UNSUPPORTED;
  if (m->lay.kind == VS_STRIPED1) return VS_ERR_UNSUPPORTED;
  return launch_attn_fwd_packed(q.dtype, view(q), view(k), view(v), m, scale, o, lse, accumulate, status,
                                (hipStream_t)stream);
}

int vs_merge_lse(float* o_acc, float* lse_acc, const float* o_step, const float* lse_step, int Hq, int64_t Nq,
                 int D, void* stream) {
  if (!o_acc || !lse_acc || !o_step || !lse_step || Hq <= 0 || Nq < 0) return VS_ERR_ARG;
  if (D != 64 && D != 128) return VS_ERR_UNSUPPORTED;
  if (!aligned16(o_acc) || !aligned16(o_step)) return VS_ERR_UNSUPPORTED;
  if (Nq == 0) return VS_OK;
  return launch_merge(o_acc, lse_acc, o_step, lse_step, Hq, Nq, D, (hipStream_t)stream);
}

int vs_convert_f16(const void* src, void* dst, int64_t n, int32_t* status, void* stream) {
  if (!src || !dst || !status || n < 0) return VS_ERR_ARG;
  if (!aligned16(src) || !aligned16(dst) || n % 8) return VS_ERR_UNSUPPORTED;
  if (n == 0) return VS_OK;
  return launch_convert_f16(src, dst, n, status, (hipStream_t)stream);
}

int vs_attn_bwd_prep(const float* o, vs_tensor dout, float* delta, void* stream) {
  if (!o || !delta || !dout.ptr) return VS_ERR_ARG;
  int st;
  if ((st = check_tensor(dout, dout.H, dout.N, dout.D)) != VS_OK) return st;
  if (!supported_attn_dtype_dim(dout.dtype, dout.D)) return VS_ERR_UNSUPPORTED;
  if (!aligned16(o)) return VS_ERR_UNSUPPORTED;
  if (dout.H <= 0 || dout.N <= 0) return VS_ERR_ARG;
  return launch_bwd_prep(o, dout.dtype, view(dout), dout.H, dout.N, dout.D, delta, (hipStream_t)stream);
}

int vs_attn_bwd_prep_f16(const float* o, const void* dout, void* dout_f16, int Hq, int64_t Nq, int D, float* delta,
                         int32_t* status, void* stream) {
  if (!o || !dout || !dout_f16 || !delta || !status || Hq <= 0 || Nq <= 0) return VS_ERR_ARG;
  if (D != 128 && D != 64) return VS_ERR_UNSUPPORTED;
  if (!aligned16(o) || !aligned16(dout) || !aligned16(dout_f16)) return VS_ERR_UNSUPPORTED;
  return launch_bwd_prep_f16(o, dout, dout_f16, Hq, Nq, D, delta, status, (hipStream_t)stream);
}

int vs_attn_bwd_parts(vs_tensor q, vs_tensor k, vs_tensor v, vs_tensor dout, const float* lse, const float* delta,
                      const vs_mask* m, float scale, float* dq, float* dk, float* dv, int parts, void* stream) {
  int st;
  if ((st = check_attn(q, k, v, m)) != VS_OK) return st;
  if ((st = check_tensor(dout, m->Hq, (int64_t)m->QB * 64, q.D)) != VS_OK) return st;
  if (dout.dtype != q.dtype) return VS_ERR_ARG;
  if ((parts & VS_BWD_ALL) == 0 || (parts & ~(VS_BWD_ALL | VS_BWD_OVERWRITE))) return VS_ERR_ARG;
  if (!lse || !delta || !dq || !dk || !dv) return VS_ERR_ARG;
  if (!aligned16(dq) || !aligned16(dk) || !aligned16(dv)) return VS_ERR_UNSUPPORTED;
  if (!finite_positive(scale)) return VS_ERR_ARG;
  return launch_attn_bwd(q.dtype, q.D, view(q), view(k), view(v), view(dout), lse, delta, m, scale, dq, dk, dv,
                         parts, (hipStream_t)stream);
}

int vs_attn_bwd(vs_tensor q, vs_tensor k, vs_tensor v, vs_tensor dout, const float* lse, const float* delta,
                const vs_mask* m, float scale, float* dq, float* dk, float* dv, void* stream) {
  return vs_attn_bwd_parts(q, k, v, dout, lse, delta, m, scale, dq, dk, dv, VS_BWD_ALL, stream);
}

// One rank's ring steps: every mask describes the same rank and layout, the
// steps see distinct shards, and K/V hold every shard in storage order.
static int check_ring(const vs_tensor& q, const vs_tensor& k, const vs_tensor& v, const vs_mask* ms, int nsteps) {
  int st;
  if (!ms || nsteps < 1) return VS_ERR_ARG;
  const vs_mask& m = ms[0];
  if (!m.tile_ptr || m.rank < 0) return VS_ERR_ARG;
  const int P = m.lay.P;
  if (nsteps > P) return VS_ERR_ARG;
  uint64_t seen[64] = {};
  if (P > 64 * 64) return VS_ERR_UNSUPPORTED;
  for (int s = 0; s < nsteps; ++s) {
    const vs_mask& x = ms[s];
    if (!x.tile_ptr || !x.tile_col || !x.csc_ptr || !x.csc_row || !x.vloc || !x.vloc_cnt || !x.vcum ||
        !x.vert_end || !x.slash_bits)
      return VS_ERR_ARG;
    if (x.Hq != m.Hq || x.Hkv != m.Hkv || x.QB != m.QB || x.KB != m.KB || x.T != m.T || x.W != m.W ||
        x.lay.kind != m.lay.kind || x.lay.P != P || x.lay.n_global != m.lay.n_global || x.rank != m.rank ||
        x.tile_cap != m.tile_cap)
      return VS_ERR_ARG;
    if (x.src < 0 || x.src >= P) return VS_ERR_ARG;
    if (seen[x.src >> 6] & (1ull << (x.src & 63))) return VS_ERR_ARG;   // each shard once
    seen[x.src >> 6] |= 1ull << (x.src & 63);
  }
  const int D = q.D;
  const int64_t Nq = (int64_t)m.QB * 64, Nall = (int64_t)P * m.KB * 64;
  if ((st = check_tensor(q, m.Hq, Nq, D)) != VS_OK) return st;
  if ((st = check_tensor(k, m.Hkv, Nall, D)) != VS_OK) return st;
  if ((st = check_tensor(v, m.Hkv, Nall, D)) != VS_OK) return st;
  if (q.dtype != k.dtype || q.dtype != v.dtype) return VS_ERR_ARG;
  if ((q.dtype != VS_BF16 && q.dtype != VS_F16) || D != 128) return VS_ERR_UNSUPPORTED;
  if (m.lay.kind == VS_STRIPED1) return VS_ERR_UNSUPPORTED;
  return VS_OK;
}

int vs_attn_fwd_ring(vs_tensor q, vs_tensor k_all, vs_tensor v_all, const vs_mask* masks, int nsteps, float scale,
                     float* o, float* lse, int accumulate, void* stream) {
  int st;
  if ((st = check_ring(q, k_all, v_all, masks, nsteps)) != VS_OK) return st;
  if (!o || !lse || !aligned16(o)) return VS_ERR_ARG;
  if (accumulate != 0 && accumulate != 1) return VS_ERR_ARG;
  if (!finite_positive(scale)) return VS_ERR_ARG;
  return launch_attn_fwd_ring(q.dtype, view(q), view(k_all), view(v_all), masks, nsteps, scale, o, lse, accumulate,
                              (hipStream_t)stream);
}

int vs_attn_bwd_ring(vs_tensor q, vs_tensor k_all, vs_tensor v_all, vs_tensor dout, const float* lse,
                     const float* delta, const vs_mask* masks, int nsteps, float scale, float* dq, float* dk_all,
                     float* dv_all, int parts, void* stream) {
  int st;
  if ((st = check_ring(q, k_all, v_all, masks, nsteps)) != VS_OK) return st;
  if ((st = check_tensor(dout, masks[0].Hq, (int64_t)masks[0].QB * 64, q.D)) != VS_OK) return st;
  if (dout.dtype != q.dtype) return VS_ERR_ARG;
  if ((parts & VS_BWD_ALL) == 0 || (parts & ~(VS_BWD_ALL | VS_BWD_OVERWRITE))) return VS_ERR_ARG;
  if (!lse || !delta || !dq || !dk_all || !dv_all) return VS_ERR_ARG;
  if (!aligned16(dq) || !aligned16(dk_all) || !aligned16(dv_all)) return VS_ERR_UNSUPPORTED;
  if (!finite_positive(scale)) return VS_ERR_ARG;
  return launch_attn_bwd_ring(q.dtype, view(q), view(k_all), view(v_all), view(dout), lse, delta, masks, nsteps,
                              scale, dq, dk_all, dv_all, parts, (hipStream_t)stream);
}

}  // extern "C"
