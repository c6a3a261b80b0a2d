// C entry points of liblce03 (declared in include/flce.h): argument
// validation, the chunk planner, workspace carving and the launch sequence.
//
// FLCE (torchtune + Liger blog, Figure 1 text; liger-kernel README,
// FusedLinearCrossEntropy): for each chunk of rows,
//   1. logits GEMM     Z_c = X_c W^T (+ b)        -> workspace chunk buffer
//   2. row CE          loss rows; Z_c := dZ_c in place
//   3. bias colsum     grad_bias (+)= column sums of dZ_c
//   4. grad_W GEMM     grad_W (+)= dZ_c^T X_c
//   5. grad_X GEMM     grad_X[c rows] = dZ_c W
// followed by one deterministic loss reduction. Everything is enqueued on the
// caller's stream; nothing is allocated.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <mutex>
#include <vector>

#include "../../include/flce.h"
#include "lce_common.h"

using namespace lce;

namespace {

constexpr size_t kAlign = 256;
constexpr size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
inline size_t elem_bytes(int dtype) { return dtype == FLCE_F32 ? 4 : 2; }
inline bool is16(int dtype) { return dtype == FLCE_BF16 || dtype == FLCE_F16; }
inline bool valid_dtype(int dtype) { return dtype == FLCE_F32 || is16(dtype); }

// The 16-bit GEMMs address a 256-row tile of an operand or of the chunk
// buffer with 32-bit byte offsets: row strides (H, and the chunk stride
// round_up(V, 8)) must stay below 2^22 elements.
constexpr int64_t kMax16Stride = int64_t(1) << 22;
inline bool gemm16_fits(int dtype, int64_t H, int64_t V) {
  return !is16(dtype) || (H < kMax16Stride && round_up(V, 8) < kMax16Stride);
}

// The GEMM for the call's element type.
inline hipError_t gemm_for(int dtype, const GemmDesc& d, hipStream_t s) {
  return is16(dtype) ? launch_gemm_16(d, dtype == FLCE_F16, s) : launch_gemm_f32(d, s);
}
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Scaling of the gradients in the chunk buffer: fp16 dlogits are stored times
// 2^kF16GradShift and without the reduction's scale (hdr->scale, or nothing
// when the rows carry their own factors: hdr == null), which the gradient
// GEMMs and column sums apply in fp32; other types store the scaled gradient.
struct GradScaling {
  int row_shift;           // grad_shift of the row kernel
  const float* out_scale;  // consumers' device factor (null: 1)
  int out_shift;           // consumers' power-of-two factor 2^-out_shift
};
// `bound` bounds the row kernel's factor before the shift (1 for the CE
// rows, beta / P for DPO's per-row factors, 1 / T for distillation); the
// shift is the largest that keeps bound * 2^shift within 2^kF16GradShift, so
// the stored values stay finite in fp16 (at least 1).
inline GradScaling grad_scaling(int dtype, const WsHeader* hdr, double bound = 1.0) {
  if (dtype != FLCE_F16) return {0, nullptr, 0};
  const double cap = std::ldexp(1.0, kF16GradShift);
  int shift = 1;
  while (shift < 30 && std::ldexp(bound, shift + 1) <= cap) ++shift;
  return {shift, hdr != nullptr ? &hdr->scale : nullptr, shift};
}
inline void scale_output(GemmDesc& d, const GradScaling& g) {
  d.out_scale = g.out_scale;
  d.out_shift = g.out_shift;
}

#ifndef LCE_LAST_SPLITS
#define LCE_LAST_SPLITS 2
#endif

constexpr int64_t kMaxRows = int64_t(1) << 31;     // int32 row indices
// Rows of one launch of a one-workgroup-per-row kernel: 1024-lane workgroups
// keep a launch within 2^32 - 1 work-items. Standalone calls (a launch over
// all N rows) are limited to this; FLCE chunks are clamped to it.
constexpr int64_t kMaxLaunchRows = (int64_t(1) << 22) - 1;
constexpr int64_t kMaxDim = int64_t(1) << 30;
// Default byte budget of one chunk's logits (the planner's only memory knob).
constexpr double kChunkBudget = 2.4e9;
constexpr int64_t kRowQuantum = 256;  // GEMM tile rows
constexpr int64_t kMinChunkRows = 8192;
// Standalone CE and shard-statistics calls up to this many rows count their
// targets inside the row kernel (each workgroup reads all of them: 8 KiB).
constexpr int64_t kSelfCountRows = 2048;

struct Plan {
  int64_t chunk;    // rows per chunk
  int64_t ldz;      // row stride of the chunk buffer (elements)
  int dx_splits;    // K-splits of the grad_X GEMM
  int last_splits;  // K-splits of the last chunk's grad_X GEMM when packed
  size_t off_rows;  // per-row losses [N] float
  size_t off_chunk; // chunk buffer [chunk, ldz]
  size_t off_split; // split-K partials [S, chunk, H] float, S = the largest split used
                    // (present when S > 1, and always for 16-bit inputs)
  // Row packing (16-bit inputs): packed-row map [N], packed targets [N] and
  // the pack kernels' block counts. The chunk's gathered hidden states
  // [chunk, H] (16-bit, half a split's bytes) sit at the start of the split-K
  // partials: each chunk's grad_W product, their last reader, runs before its
  // grad_X product writes partials. pack_ok is false for float32 inputs.
  bool pack_ok;
  size_t off_map, off_ptgt, off_bcnt, off_xs;
  // When the rest of the split-K partials holds it too: the gathered rows
  // transposed, [H, ldt] (ldt = chunk rounded up to 64), the k-contiguous B
  // operand of the grad_W product.
  bool xt_ok;
  int64_t ldt;
  size_t off_xt;
  size_t total;
};

// Choose the K-split count of grad_X = dZ_c W (M = chunk, N = H, K = V) that
// best fills whole waves of 256 workgroups (one 256x256 tile per CU).
int choose_dx_splits(int64_t chunk, int64_t H, int64_t V) {
  const int64_t tiles = ((chunk + 255) / 256) * ((H + 255) / 256);
  auto fill = [&](int s) {
    const int64_t units = tiles * s;
    const int64_t waves = (units + 255) / 256;
    return static_cast<double>(units) / static_cast<double>(waves * 256);
  };
  // A split must keep at least 2048 of K and must raise the fill by > 2%.
  int best = 1;
  double best_eff = fill(1);
  for (int s = 2; s <= 8; s *= 2) {
    if (V / s < 2048) break;
    const double eff = fill(s);
    if (eff > best_eff + 0.02) { best_eff = eff; best = s; }
  }
  return best;
}

bool make_plan(int64_t N, int64_t H, int64_t V, int dtype, int64_t chunk_rows, Plan* p) {
  if (N < 0 || H <= 0 || V <= 0 || N >= kMaxRows || H >= kMaxDim || V >= kMaxDim) return false;
  if (!valid_dtype(dtype)) return false;
  if (chunk_rows < 0) return false;
  const size_t e = elem_bytes(dtype);
  const int64_t ldz = round_up(V, 8);
  int64_t chunk;
  if (chunk_rows > 0) {
    chunk = std::min(std::min(chunk_rows, std::max<int64_t>(N, 1)), kMaxLaunchRows);
  } else {
    // Largest multiple of 256 rows under the budget, then evened out over
    // the chunks; never one chunk holding every row of a multi-tile batch,
    // so the [N, V] logits are never materialised.
    int64_t cmax = static_cast<int64_t>(kChunkBudget / (static_cast<double>(ldz) * e));
    // The grad_W product reads and rewrites the float32 [V, H] gradient once
    // per chunk, so its K (the chunk's rows) should not be short: up to twice
    // the budget is spent to reach kMinChunkRows.
    if (cmax < kMinChunkRows)
      cmax = std::min<int64_t>(kMinChunkRows,
                               static_cast<int64_t>(2.0 * kChunkBudget / (static_cast<double>(ldz) * e)));
    cmax = std::max<int64_t>(kRowQuantum, cmax / kRowQuantum * kRowQuantum);
    if (N > 2 * kRowQuantum) cmax = std::min(cmax, round_up((N + 1) / 2, kRowQuantum));
    const int64_t n1 = std::max<int64_t>(N, 1);
    if (cmax >= n1) {
      chunk = n1;
    } else {
      const int64_t nchunks = (n1 + cmax - 1) / cmax;
      chunk = std::min(round_up((n1 + nchunks - 1) / nchunks, kRowQuantum), cmax);
    }
  }
  p->chunk = chunk;
  p->ldz = ldz;
  p->dx_splits = is16(dtype) ? choose_dx_splits(chunk, H, V) : 1;
  // Packed, the last chunk usually holds fewer live rows than the others;
  // its grad_X tiles (256 rows x 256 columns) then fill the CUs unevenly, and
  // splitting K in two halves the granularity.
  p->last_splits = p->dx_splits;
  if (is16(dtype))
    while (p->last_splits < LCE_LAST_SPLITS && V / (2 * p->last_splits) >= 2048) p->last_splits *= 2;
  // Packed heads that add to grad_X reduce it through the partial buffer
  // (one split), so 16-bit plans always hold at least one.
  const int max_splits = std::max(std::max(p->dx_splits, p->last_splits), is16(dtype) ? 1 : 0);
  size_t off = align_up(sizeof(WsHeader));
  p->off_rows = off;
  off += align_up(static_cast<size_t>(std::max<int64_t>(N, 1)) * sizeof(float));
  p->off_chunk = off;
  off += align_up(static_cast<size_t>(chunk) * static_cast<size_t>(ldz) * e);
  p->off_split = off;
  if (max_splits > 1 || is16(dtype))
    off += align_up(static_cast<size_t>(max_splits) * static_cast<size_t>(chunk) *
                    static_cast<size_t>(H) * sizeof(float));
  p->pack_ok = is16(dtype);
  p->off_xs = p->off_split;
  {
    const size_t split_bytes = off - p->off_split;
    const size_t xs_bytes = align_up(static_cast<size_t>(chunk) * static_cast<size_t>(H) * e);
    p->ldt = round_up(chunk, 64);
    p->off_xt = p->off_split + xs_bytes;
    p->xt_ok = p->pack_ok && p->ldt < kMax16Stride &&
               xs_bytes + static_cast<size_t>(H) * static_cast<size_t>(p->ldt) * e <= split_bytes;
  }
  p->off_map = p->off_ptgt = p->off_bcnt = off;
  if (p->pack_ok) {
    const size_t n1 = static_cast<size_t>(std::max<int64_t>(N, 1));
    p->off_map = off;
    off += align_up(n1 * sizeof(int32_t));
    p->off_ptgt = off;
    off += align_up(n1 * sizeof(int32_t));
    p->off_bcnt = off;
    off += align_up(static_cast<size_t>(std::max<int64_t>(pack_block_count(N), 1)) * sizeof(int32_t));
  }
  p->total = off;
  return true;
}

constexpr size_t ce_ws_bytes(int64_t N) {
  return align_up(sizeof(WsHeader)) + align_up(static_cast<size_t>(std::max<int64_t>(N, 1)) * sizeof(float));
}

// ------------------------------------------------------------- timing

struct TimedLaunch {
  int kind;
  hipEvent_t start, stop;
};
bool g_timing = false;
std::vector<TimedLaunch> g_records;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t take_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Runs `launch` on stream s, bracketed by events when timing is on.
template <typename F>
hipError_t timed(int kind, hipStream_t s, F&& launch) {
  if (!g_timing) return launch();
  TimedLaunch r{kind, take_event(), take_event()};
  if (r.start == nullptr || r.stop == nullptr) return hipErrorOutOfMemory;
  hipError_t e = hipEventRecord(r.start, s);
  if (e != hipSuccess) return e;
  e = launch();
  if (e != hipSuccess) return e;
  e = hipEventRecord(r.stop, s);
  if (e != hipSuccess) return e;
  g_records.push_back(r);
  return hipSuccess;
}

enum Kind { kKindLogits = 0, kKindRowCE = 1, kKindGradX = 2, kKindGradW = 3, kKindOther = 4 };

// Row packing switch (flce_set_row_packing); on by default.
bool g_row_packing = true;

#define LCE_TRY(expr)                          \
  do {                                         \
    if ((expr) != hipSuccess) return FLCE_E_HIP; \
  } while (0)

}  // namespace

extern "C" {

const char* flce_status_string(int status) {
  switch (status) {
    case FLCE_OK: return "ok";
    case FLCE_E_INVALID_ARG: return "invalid argument (null pointer, size, enum or shape)";
    case FLCE_E_WORKSPACE: return "workspace missing or smaller than required";
    case FLCE_E_UNSUPPORTED: return "unsupported layout (pointer not 16-byte aligned, bf16 H not a multiple of 8, or size limit)";
    case FLCE_E_TARGET: return "a target outside [0, V) that is not ignore_index";
    case FLCE_E_HIP: return "HIP runtime or kernel launch error";
    default: return "unknown status";
  }
}

size_t flce_workspace_bytes(int64_t N, int64_t H, int64_t V, int dtype, int64_t chunk_rows) {
  Plan p;
  if (!make_plan(N, H, V, dtype, chunk_rows, &p)) return 0;
  return p.total;
}

int flce_plan(int64_t N, int64_t H, int64_t V, int dtype, int64_t chunk_rows, int64_t* chunk_rows_out,
              int32_t* dx_splits_out) {
  Plan p;
  if (!make_plan(N, H, V, dtype, chunk_rows, &p)) return FLCE_E_INVALID_ARG;
  if (chunk_rows_out) *chunk_rows_out = p.chunk;
  if (dx_splits_out) *dx_splits_out = p.dx_splits;
  return FLCE_OK;
}

int flce_workspace_parts(int64_t N, int64_t H, int64_t V, int dtype, int64_t chunk_rows,
                         size_t* parts) {
  Plan p;
  if (parts == nullptr || !make_plan(N, H, V, dtype, chunk_rows, &p)) return FLCE_E_INVALID_ARG;
  parts[0] = p.off_chunk;                  // header + per-row losses
  parts[1] = p.off_split - p.off_chunk;    // chunk logits / dlogits
  parts[2] = p.off_map - p.off_split;      // grad_X K-split partials (and gathered rows)
  parts[3] = p.total - p.off_map;          // packed-row lists
  return FLCE_OK;
}

int flce_set_row_packing(int enable) {
  const int was = g_row_packing ? 1 : 0;
  g_row_packing = enable != 0;
  return was;
}

size_t ce_workspace_bytes(int64_t N, int64_t V) {
  if (N < 0 || V <= 0 || N >= kMaxRows || V >= kMaxDim) return 0;
  return ce_ws_bytes(N);
}

static int validate_common(int dtype, int reduction) {
  if (!valid_dtype(dtype)) return FLCE_E_INVALID_ARG;
  if (reduction < FLCE_REDUCTION_NONE || reduction > FLCE_REDUCTION_MEAN) return FLCE_E_INVALID_ARG;
  return FLCE_OK;
}

}  // extern "C"

namespace {

// Row packing state of one call's chunk loop (see flce_chunks).
struct Packer {
  bool on = false;
  int32_t* map = nullptr;          // packed row -> original row [N]
  const int32_t* ptgt = nullptr;   // packed targets [N]
  char* xs = nullptr;              // the chunk's gathered hidden states [chunk, H]
  char* xt = nullptr;              // ... and transposed [H, ldt] (when t_on)
  int64_t ldt = 0;
  bool t_on = false;
  const int32_t* live = nullptr;   // &hdr->n_packed

  // Lists the rows whose target is valid against V_valid, zeroes the other
  // rows' loss entries (loss_rows may be null) and, when grad_X is given,
  // their grad_X rows of gx_row_bytes bytes.
  int setup(const Plan& p, char* ws, WsHeader* hdr, const int32_t* targets, int64_t N,
            int64_t V_valid, int32_t ign, float* loss_rows, void* grad_X, int64_t gx_row_bytes,
            hipStream_t s, bool allow = true, bool allow_t = true) {
    on = allow && g_row_packing && p.pack_ok && N > 0;
    if (!on) return FLCE_OK;
    map = reinterpret_cast<int32_t*>(ws + p.off_map);
    ptgt = reinterpret_cast<const int32_t*>(ws + p.off_ptgt);
    xs = ws + p.off_xs;
    t_on = allow_t && p.xt_ok;
    xt = ws + p.off_xt;
    ldt = p.ldt;
    live = &hdr->n_packed;
    LCE_TRY(timed(kKindOther, s, [&] {
      return launch_pack_rows(targets, N, V_valid, ign, map, const_cast<int32_t*>(ptgt),
                              reinterpret_cast<int32_t*>(ws + p.off_bcnt), hdr, loss_rows, s);
    }));
    if (grad_X)
      LCE_TRY(timed(kKindOther, s, [&] {
        return launch_zero_dead_rows(targets, N, V_valid, ign, grad_X, gx_row_bytes, s);
      }));
    return FLCE_OK;
  }
  RowPack chunk(int64_t r0) const {
    return on ? RowPack{map + r0, live, r0} : RowPack{nullptr, nullptr, 0};
  }
  // The chunk's rows of X: gathered when packed, else rows r0.. of X. With
  // Xt given and the plan holding it, also their transpose (*Xt, else null).
  int rows_of(const void* X, int64_t r0, int64_t rows, int64_t H, size_t e, hipStream_t s,
              const char** Xc, const char** Xt = nullptr) const {
    *Xc = static_cast<const char*>(X) + static_cast<size_t>(r0) * H * e;
    if (Xt) *Xt = nullptr;
    if (!on) return FLCE_OK;
    if (Xt && t_on) {
      LCE_TRY(timed(kKindOther, s, [&] {
        return launch_gather_rows_t(X, H, rows, chunk(r0), xs, xt, ldt, s);
      }));
      *Xt = xt;
    } else {
      LCE_TRY(timed(kKindOther, s, [&] {
        return launch_gather_rows(X, H * static_cast<int64_t>(e), rows, chunk(r0), xs, s);
      }));
    }
    *Xc = xs;
    return FLCE_OK;
  }
  // A GEMM whose M (dim 0) or K (dim 1) runs over the chunk's rows.
  void limit(GemmDesc& d, int dim, int64_t r0) const {
    if (!on) return;
    d.live = live; d.live_base = r0; d.live_dim = dim;
  }
};

// The two gradient products of one chunk whose dlogits are in zbuf:
//   grad_W = dZ_c^T X_c (stored on the first chunk, added after), reading
//   the transposed gathered rows Xt ([H, ldt], k-contiguous) when given;
//   grad_X rows = dZ_c W (stored, or added when accum_gx), W read as stored
//   (n-major B operand).
// grad_W runs first: it is the last reader of the chunk's gathered rows,
// which share the split-K partial buffer that grad_X may write. The last
// packed chunk's grad_X is split along K (its part-full tile rounds are then
// half as long). grad_X goes through the split-K partial buffer when it is
// split, or when a packed chunk adds to grad_X (the reduction then adds each
// row to its original row). Either gradient may be null.
int gradient_products(const Plan& p, int dtype, const void* W, int64_t H, int64_t V, void* zbuf,
                      const char* Xc, const char* Xt, int64_t rows, int64_t r0, int64_t N, bool first,
                      const Packer& pkr, const RowPack& pk, void* grad_X, bool accum_gx,
                      void* grad_W, int grad_dtype, const GradScaling& gsc, char* ws,
                      hipStream_t s) {
  const bool g16 = grad_dtype != FLCE_F32;
  const size_t ge = g16 ? 2 : 4;
  const bool pack = pkr.on;
  float* split_buf = reinterpret_cast<float*>(ws + p.off_split);
  auto gemm = [dtype](const GemmDesc& d, hipStream_t st) { return gemm_for(dtype, d, st); };
  if (grad_W) {
    GemmDesc g3{};
    g3.A = zbuf; g3.lda = p.ldz; g3.a_kmajor = false;
    if (Xt) {
      g3.B = Xt; g3.ldb = p.ldt; g3.b_kmajor = true;
    } else {
      g3.B = Xc; g3.ldb = H; g3.b_kmajor = false;
    }
    g3.C = grad_W; g3.ldc = H;
    g3.M = V; g3.N = H; g3.K = rows;
    g3.epilogue = first ? (g16 ? kEpiStore16 : kEpiStoreF32) : (g16 ? kEpiAccum16 : kEpiAccumF32);
    g3.k_splits = 1;
    scale_output(g3, gsc);
    pkr.limit(g3, 1, r0);
    LCE_TRY(timed(kKindGradW, s, [&] { return gemm(g3, s); }));
  }
  if (grad_X) {
    GemmDesc g2{};
    g2.A = zbuf; g2.lda = p.ldz; g2.a_kmajor = true;
    g2.B = W; g2.ldb = H; g2.b_kmajor = false;
    g2.M = rows; g2.N = H; g2.K = V;
    scale_output(g2, gsc);
    pkr.limit(g2, 0, r0);
    void* out = static_cast<char*>(grad_X) + (pack ? 0 : static_cast<size_t>(r0) * H * ge);
    const int splits = (pack && r0 + p.chunk >= N) ? p.last_splits : p.dx_splits;
    const bool via_split = splits > 1 || (pack && accum_gx);
    if (via_split) {
      g2.epilogue = kEpiStoreF32;
      g2.C = split_buf; g2.ldc = H;
      g2.k_splits = splits; g2.split_stride = rows * H;
    } else {
      g2.epilogue = accum_gx ? (g16 ? kEpiAccum16 : kEpiAccumF32) : (g16 ? kEpiStore16 : kEpiStoreF32);
      g2.C = out; g2.ldc = H; g2.k_splits = 1;
      if (pack) g2.row_map = pk.map;
    }
    LCE_TRY(timed(kKindGradX, s, [&] { return gemm(g2, s); }));
    if (via_split)
      LCE_TRY(timed(kKindOther, s, [&] {
        return launch_splitk_reduce(split_buf, splits, rows * H, rows, H, H, out, grad_dtype,
                                    accum_gx, s, pk);
      }));
  }
  return FLCE_OK;
}

// The chunk loop of FLCE over all N rows for one head: logits GEMM, row CE
// (loss rows, dZ in place), bias column sums, grad_X (stored, or added to
// what is there when accum_gx), grad_W (stored on the first chunk, added
// after). Targets must have been counted into hdr.
//
// Row packing (16-bit inputs): rows with an ignored or
// invalid target contribute nothing, so they are listed out first and every
// chunk covers the next `chunk` of the remaining rows. The host does not know
// how many remain (the count lives on the device and is never read back), so
// it launches every chunk for `chunk` rows and the kernels stop at the live
// count: GEMM tiles past it exit, the grad_W product shortens its K loop. The
// chunk's hidden states are gathered into the workspace for the logits and
// grad_W products; loss and grad_X rows are written back to their original
// rows, and grad_X rows of the dropped rows are zeroed (or, when adding to
// grad_X, left as they are: the chunk's partial products then go through the
// split-K buffer and its reduction adds them to the original rows).
int flce_chunks(const Plan& p, int dtype, const void* X, const void* W, const void* bias,
                const int32_t* targets, int64_t N, int64_t H, int64_t V, int32_t ignore_index,
                WsHeader* hdr, float* loss_rows, void* grad_X, bool accum_gx, void* grad_W,
                void* grad_bias, int grad_dtype, char* ws, hipStream_t s) {
  // grad_dtype: FLCE_F32, or the 16-bit input type (gradients rounded to it;
  // grad_W and grad_bias are accumulated across chunks in that type).
  const bool g16 = grad_dtype != FLCE_F32;
  const size_t ge = g16 ? 2 : 4;
  void* zbuf = ws + p.off_chunk;
  const size_t e = elem_bytes(dtype);
  const bool need_grad = grad_X != nullptr || grad_W != nullptr || grad_bias != nullptr;
  auto gemm = [dtype](const GemmDesc& d, hipStream_t st) { return gemm_for(dtype, d, st); };
  const GradScaling gsc = grad_scaling(dtype, hdr);

  Packer pkr;
  int st = pkr.setup(p, ws, hdr, targets, N, V, ignore_index, loss_rows,
                     accum_gx ? nullptr : grad_X, H * static_cast<int64_t>(ge), s);
  if (st != FLCE_OK) return st;
  const bool pack = pkr.on;
  const int32_t* ptgt = pkr.ptgt;

  for (int64_t r0 = 0; r0 < N; r0 += p.chunk) {
    const int64_t rows = std::min(p.chunk, N - r0);
    const bool first = r0 == 0;
    // Packed: chunk rows are packed rows r0.. (live up to hdr->n_packed).
    const RowPack pk = pkr.chunk(r0);
    const char *Xc, *Xt;
    st = pkr.rows_of(X, r0, rows, H, e, s, &Xc, grad_W ? &Xt : nullptr);
    if (st != FLCE_OK) return st;
    if (!grad_W) Xt = nullptr;
    auto live = [&](GemmDesc& d, int dim) { pkr.limit(d, dim, r0); };

    GemmDesc g1{};
    g1.A = Xc; g1.lda = H; g1.a_kmajor = true;
    g1.B = W; g1.ldb = H; g1.b_kmajor = true;
    g1.C = zbuf; g1.ldc = p.ldz; g1.bias = bias;
    g1.M = rows; g1.N = V; g1.K = H;
    g1.epilogue = kEpiLogits; g1.k_splits = 1;
    live(g1, 0);
    LCE_TRY(timed(kKindLogits, s, [&] { return gemm(g1, s); }));

    LCE_TRY(timed(kKindRowCE, s, [&] {
      return launch_row_ce(dtype, zbuf, p.ldz, need_grad ? zbuf : nullptr, p.ldz, rows, V,
                           p.ldz - V, (pack ? ptgt : targets) + r0, ignore_index, hdr,
                           pack ? loss_rows : loss_rows + r0, nullptr, gsc.row_shift, s, pk);
    }));
    if (!need_grad) continue;

    if (grad_bias)
      LCE_TRY(timed(kKindOther, s, [&] {
        return launch_colsum(dtype, zbuf, p.ldz, rows, V, grad_bias, grad_dtype, !first,
                             gsc.out_scale, gsc.out_shift, s, pk);
      }));

    st = gradient_products(p, dtype, W, H, V, zbuf, Xc, Xt, rows, r0, N, first, pkr, pk, grad_X,
                           accum_gx, grad_W, grad_dtype, gsc, ws, s);
    if (st != FLCE_OK) return st;
  }
  return FLCE_OK;
}

// Validation shared by the single- and multi-head calls.
int validate_flce(const void* X, const void* W, const void* bias, const int32_t* targets,
                  int64_t N, int64_t H, int64_t V, int dtype, int reduction, const float* loss,
                  const void* grad_X, const void* grad_W, const void* grad_bias,
                  int64_t chunk_rows, const void* workspace) {
  int st = validate_common(dtype, reduction);
  if (st != FLCE_OK) return st;
  if (N < 0 || H <= 0 || V <= 0 || chunk_rows < 0) return FLCE_E_INVALID_ARG;
  if (W == nullptr || loss == nullptr) return FLCE_E_INVALID_ARG;
  if (N > 0 && (X == nullptr || targets == nullptr)) return FLCE_E_INVALID_ARG;
  if (grad_bias != nullptr && bias == nullptr) return FLCE_E_INVALID_ARG;
  if (N >= kMaxRows || H >= kMaxDim || V >= kMaxDim) return FLCE_E_UNSUPPORTED;
  const void* ptrs[] = {X, W, bias, targets, loss, grad_X, grad_W, grad_bias, workspace};
  for (const void* q : ptrs)
    if (q != nullptr && !aligned16(q)) return FLCE_E_UNSUPPORTED;
  if (is16(dtype) && (H % 8) != 0) return FLCE_E_UNSUPPORTED;
  if (!gemm16_fits(dtype, H, V)) return FLCE_E_UNSUPPORTED;
  return FLCE_OK;
}

// Per-head counters and loss rows of the multi-head call, after the FLCE plan.
size_t head_slot_bytes(int64_t N) {
  return align_up(sizeof(WsHeader)) + align_up(static_cast<size_t>(std::max<int64_t>(N, 1)) * sizeof(float));
}

int flce_forward_backward_impl(const void* X, const void* W, const void* bias,
                               const int32_t* targets, int64_t N, int64_t H, int64_t V, int dtype,
                               int32_t ignore_index, int reduction, int grad_dtype, float* loss,
                               void* grad_X, void* grad_W, void* grad_bias, void* workspace,
                               size_t workspace_bytes, int64_t chunk_rows, void* stream) {
  int st = validate_flce(X, W, bias, targets, N, H, V, dtype, reduction, loss, grad_X, grad_W,
                         grad_bias, chunk_rows, workspace);
  if (st != FLCE_OK) return st;
  if (grad_dtype != FLCE_F32 && grad_dtype != dtype) return FLCE_E_INVALID_ARG;
  Plan p;
  if (!make_plan(N, H, V, dtype, chunk_rows, &p)) return FLCE_E_INVALID_ARG;
  if (workspace == nullptr || workspace_bytes < p.total) return FLCE_E_WORKSPACE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  WsHeader* hdr = reinterpret_cast<WsHeader*>(ws);
  float* loss_rows = reduction == FLCE_REDUCTION_NONE ? loss : reinterpret_cast<float*>(ws + p.off_rows);

  LCE_TRY(timed(kKindOther, s, [&] {
    return launch_count_targets(targets, N, V, ignore_index, reduction, hdr, s);
  }));
  if (N == 0) {
    if (grad_W) LCE_TRY(timed(kKindOther, s, [&] { return launch_zero(grad_W, V * H, grad_dtype, s); }));
    if (grad_bias) LCE_TRY(timed(kKindOther, s, [&] { return launch_zero(grad_bias, V, grad_dtype, s); }));
  }
  st = flce_chunks(p, dtype, X, W, bias, targets, N, H, V, ignore_index, hdr, loss_rows, grad_X,
                   false, grad_W, grad_bias, grad_dtype, ws, s);
  if (st != FLCE_OK) return st;
  if (reduction != FLCE_REDUCTION_NONE)
    LCE_TRY(timed(kKindOther, s, [&] {
      return launch_reduce_loss(loss_rows, N, hdr, reduction, loss, s);
    }));
  return FLCE_OK;
}

}  // namespace

extern "C" {

int flce_forward_backward(const void* X, const void* W, const void* bias, const int32_t* targets,
                          int64_t N, int64_t H, int64_t V, int dtype, int32_t ignore_index,
                          int reduction, float* loss, float* grad_X, float* grad_W,
                          float* grad_bias, void* workspace, size_t workspace_bytes,
                          int64_t chunk_rows, void* stream) {
  return flce_forward_backward_impl(X, W, bias, targets, N, H, V, dtype, ignore_index, reduction,
                                    FLCE_F32, loss, grad_X, grad_W, grad_bias, workspace,
                                    workspace_bytes, chunk_rows, stream);
}

int flce_forward_backward_ex(const void* X, const void* W, const void* bias,
                             const int32_t* targets, int64_t N, int64_t H, int64_t V, int dtype,
                             int32_t ignore_index, int reduction, int grad_dtype, float* loss,
                             void* grad_X, void* grad_W, void* grad_bias, void* workspace,
                             size_t workspace_bytes, int64_t chunk_rows, void* stream) {
  return flce_forward_backward_impl(X, W, bias, targets, N, H, V, dtype, ignore_index, reduction,
                                    grad_dtype, loss, grad_X, grad_W, grad_bias, workspace,
                                    workspace_bytes, chunk_rows, stream);
}

size_t flce_multihead_workspace_bytes(int64_t N, int64_t H, int64_t V, int64_t K, int dtype,
                                      int64_t chunk_rows) {
  Plan p;
  if (K <= 0 || K >= kMaxDim || !make_plan(N, H, V, dtype, chunk_rows, &p)) return 0;
  return p.total + static_cast<size_t>(K) * head_slot_bytes(N);
}

}  // extern "C"

namespace {

int flce_multihead_impl(const void* X, const void* W, const void* bias, const int32_t* targets,
                        int64_t N, int64_t H, int64_t V, int64_t K, int dtype, int32_t ignore_index,
                        int reduction, int grad_dtype, float* loss, void* grad_X, void* grad_W,
                        void* grad_bias, void* workspace, size_t workspace_bytes,
                        int64_t chunk_rows, void* stream) {
  if (K <= 0 || K >= kMaxDim) return FLCE_E_INVALID_ARG;
  int st = validate_flce(X, W, bias, targets, N, H, V, dtype, reduction, loss, grad_X, grad_W,
                         grad_bias, chunk_rows, workspace);
  if (st != FLCE_OK) return st;
  if (grad_dtype != FLCE_F32 && grad_dtype != dtype) return FLCE_E_INVALID_ARG;
  Plan p;
  if (!make_plan(N, H, V, dtype, chunk_rows, &p)) return FLCE_E_INVALID_ARG;
  const size_t slot = head_slot_bytes(N);
  if (workspace == nullptr || workspace_bytes < p.total + static_cast<size_t>(K) * slot)
    return FLCE_E_WORKSPACE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const size_t e = elem_bytes(dtype);
  const size_t ge = grad_dtype == FLCE_F32 ? 4 : 2;
  // Each head counts its targets into its own slot so N_valid is per head;
  // the call's own header (the first slot of the plan) counts all K x N
  // targets, so that flce_check_device_error sees a bad target in any head.
  LCE_TRY(timed(kKindOther, s, [&] {
    return launch_count_targets(targets, K * N, V, ignore_index, reduction,
                                reinterpret_cast<WsHeader*>(ws), s);
  }));
  for (int64_t k = 0; k < K; ++k) {
    char* hs = ws + p.total + static_cast<size_t>(k) * slot;
    WsHeader* hdr = reinterpret_cast<WsHeader*>(hs);
    float* loss_rows = reduction == FLCE_REDUCTION_NONE
                           ? loss + static_cast<size_t>(k) * N
                           : reinterpret_cast<float*>(hs + align_up(sizeof(WsHeader)));
    const int32_t* tk = targets + static_cast<size_t>(k) * N;
    const char* Wk = static_cast<const char*>(W) + static_cast<size_t>(k) * V * H * e;
    const char* bk = bias ? static_cast<const char*>(bias) + static_cast<size_t>(k) * V * e : nullptr;
    void* gWk = grad_W ? static_cast<char*>(grad_W) + static_cast<size_t>(k) * V * H * ge : nullptr;
    void* gbk = grad_bias ? static_cast<char*>(grad_bias) + static_cast<size_t>(k) * V * ge : nullptr;
    LCE_TRY(timed(kKindOther, s, [&] {
      return launch_count_targets(tk, N, V, ignore_index, reduction, hdr, s);
    }));
    if (N == 0) {
      if (gWk) LCE_TRY(timed(kKindOther, s, [&] { return launch_zero(gWk, V * H, grad_dtype, s); }));
      if (gbk) LCE_TRY(timed(kKindOther, s, [&] { return launch_zero(gbk, V, grad_dtype, s); }));
    }
    st = flce_chunks(p, dtype, X, Wk, bk, tk, N, H, V, ignore_index, hdr, loss_rows, grad_X, k > 0,
                     gWk, gbk, grad_dtype, ws, s);
    if (st != FLCE_OK) return st;
    if (reduction != FLCE_REDUCTION_NONE)
      LCE_TRY(timed(kKindOther, s, [&] {
        return launch_reduce_loss(loss_rows, N, hdr, reduction, loss + k, s);
      }));
  }
  return FLCE_OK;
}

}  // namespace

extern "C" {

int flce_multihead_forward_backward(const void* X, const void* W, const void* bias,
                                    const int32_t* targets, int64_t N, int64_t H, int64_t V,
                                    int64_t K, int dtype, int32_t ignore_index, int reduction,
                                    float* loss, float* grad_X, float* grad_W, float* grad_bias,
                                    void* workspace, size_t workspace_bytes, int64_t chunk_rows,
                                    void* stream) {
  return flce_multihead_impl(X, W, bias, targets, N, H, V, K, dtype, ignore_index, reduction,
                             FLCE_F32, loss, grad_X, grad_W, grad_bias, workspace, workspace_bytes,
                             chunk_rows, stream);
}

int flce_multihead_forward_backward_ex(const void* X, const void* W, const void* bias,
                                       const int32_t* targets, int64_t N, int64_t H, int64_t V,
                                       int64_t K, int dtype, int32_t ignore_index, int reduction,
                                       int grad_dtype, float* loss, void* grad_X, void* grad_W,
                                       void* grad_bias, void* workspace, size_t workspace_bytes,
                                       int64_t chunk_rows, void* stream) {
  return flce_multihead_impl(X, W, bias, targets, N, H, V, K, dtype, ignore_index, reduction,
                             grad_dtype, loss, grad_X, grad_W, grad_bias, workspace,
                             workspace_bytes, chunk_rows, stream);
}

int ce_forward_backward(const void* logits, void* grad_logits, const int32_t* targets, int64_t N,
                        int64_t V, int dtype, int32_t ignore_index, int reduction, float* loss,
                        void* workspace, size_t workspace_bytes, void* stream) {
  int st = validate_common(dtype, reduction);
  if (st != FLCE_OK) return st;
  if (N < 0 || V <= 0 || loss == nullptr) return FLCE_E_INVALID_ARG;
  if (N > 0 && (logits == nullptr || targets == nullptr)) return FLCE_E_INVALID_ARG;
  if (N > kMaxLaunchRows || V >= kMaxDim) return FLCE_E_UNSUPPORTED;
  const void* ptrs[] = {logits, grad_logits, targets, loss, workspace};
  for (const void* q : ptrs)
    if (q != nullptr && !aligned16(q)) return FLCE_E_UNSUPPORTED;
  if (workspace == nullptr || workspace_bytes < ce_ws_bytes(N)) return FLCE_E_WORKSPACE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  WsHeader* hdr = reinterpret_cast<WsHeader*>(ws);
  float* loss_rows = reduction == FLCE_REDUCTION_NONE ? loss : reinterpret_cast<float*>(ws + align_up(sizeof(WsHeader)));
  if (N > 0 && N <= kSelfCountRows) {
    // One launch: the row kernel counts the targets itself.
    LCE_TRY(timed(kKindRowCE, s, [&] {
      return launch_row_ce_counted(dtype, logits, grad_logits, N, V, targets, ignore_index,
                                   reduction, hdr, loss_rows, s);
    }));
  } else {
    LCE_TRY(timed(kKindOther, s, [&] {
      return launch_count_targets(targets, N, V, ignore_index, reduction, hdr, s);
    }));
    LCE_TRY(timed(kKindRowCE, s, [&] {
      return launch_row_ce(dtype, logits, V, grad_logits, V, N, V, 0, targets, ignore_index, hdr,
                           loss_rows, nullptr, 0, s);
    }));
  }
  if (reduction != FLCE_REDUCTION_NONE)
    LCE_TRY(timed(kKindOther, s, [&] {
      return launch_reduce_loss(loss_rows, N, hdr, reduction, loss, s);
    }));
  return FLCE_OK;
}

}  // extern "C"

// Scratch of ce_forward_backward_noalloc: the workspace of a standalone CE
// call of up to kNoAllocMaxRows rows (the 256-byte header and one float per
// row), 16 MiB + 256 bytes per device, held until the process ends. Host code
// never passes `scratch` itself to a kernel (on the host the name is only a
// stand-in); it uses the device address that hipGetSymbolAddress returns for
// each device.
namespace {
constexpr int64_t kNoAllocMaxRows = kMaxLaunchRows;
constexpr size_t kNoAllocBytes = ce_ws_bytes(kNoAllocMaxRows);
constexpr int kMaxDevices = 64;
}  // namespace
static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the device of `stream` (looked up once
// per device, with that device current); null on a HIP error.
void* scratch_on(hipStream_t stream) {
  int dev = -1;
  if (stream != nullptr) {
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) return nullptr;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return nullptr;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return nullptr;
    if (e != hipSuccess || ptr == nullptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" {

int ce_forward_backward_noalloc(const void* logits, void* grad_logits, const int32_t* targets,
                                int64_t N, int64_t V, int dtype, int32_t ignore_index,
                                int reduction, float* loss, void* stream) {
  if (N > kNoAllocMaxRows) return FLCE_E_UNSUPPORTED;
  int st = validate_common(dtype, reduction);
  if (st != FLCE_OK) return st;
  if (N < 0 || V <= 0 || loss == nullptr) return FLCE_E_INVALID_ARG;
  if (N > 0 && (logits == nullptr || targets == nullptr)) return FLCE_E_INVALID_ARG;
  void* ws = scratch_on(static_cast<hipStream_t>(stream));
  if (ws == nullptr) return FLCE_E_HIP;
  // Same kernels as the workspace call; every header field and loss row they
  // read is written earlier in the same call, so nothing needs clearing.
  return ce_forward_backward(logits, grad_logits, targets, N, V, dtype, ignore_index, reduction,
                             loss, ws, kNoAllocBytes, stream);
}

int ce_shard_stats(const void* logits_shard, const int32_t* targets, int64_t N, int64_t V_local,
                   int64_t vocab_start, int64_t V_global, int dtype, int32_t ignore_index,
                   float* row_max, float* row_sumexp, float* row_target_logit, void* workspace,
                   size_t workspace_bytes, void* stream) {
  if (!valid_dtype(dtype)) return FLCE_E_INVALID_ARG;
  if (N < 0 || V_local <= 0 || vocab_start < 0 || V_global < vocab_start + V_local)
    return FLCE_E_INVALID_ARG;
  if (N > 0 && (logits_shard == nullptr || targets == nullptr || row_max == nullptr ||
                row_sumexp == nullptr || row_target_logit == nullptr))
    return FLCE_E_INVALID_ARG;
  if (N > kMaxLaunchRows || V_global >= kMaxDim) return FLCE_E_UNSUPPORTED;
  const void* ptrs[] = {logits_shard, targets, row_max, row_sumexp, row_target_logit, workspace};
  for (const void* q : ptrs)
    if (q != nullptr && !aligned16(q)) return FLCE_E_UNSUPPORTED;
  if (workspace == nullptr || workspace_bytes < ce_ws_bytes(N)) return FLCE_E_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  WsHeader* hdr = static_cast<WsHeader*>(workspace);
  if (N > 0 && N <= kSelfCountRows) {
    // One launch: the statistics kernel counts the targets itself.
    LCE_TRY(timed(kKindRowCE, s, [&] {
      return launch_shard_stats_counted(dtype, logits_shard, N, V_local, vocab_start, V_global,
                                        targets, ignore_index, row_max, row_sumexp,
                                        row_target_logit, hdr, s);
    }));
    return FLCE_OK;
  }
  LCE_TRY(timed(kKindOther, s, [&] {
    return launch_count_targets(targets, N, V_global, ignore_index, FLCE_REDUCTION_SUM, hdr, s);
  }));
  LCE_TRY(timed(kKindRowCE, s, [&] {
    return launch_shard_stats(dtype, logits_shard, V_local, N, V_local, vocab_start, V_global,
                              targets, ignore_index, row_max, row_sumexp, row_target_logit, s);
  }));
  return FLCE_OK;
}

int flce_shard_stats(const void* X, const void* W_shard, const void* bias_shard,
                     const int32_t* targets, int64_t N, int64_t H, int64_t V_local,
                     int64_t vocab_start, int64_t V_global, int dtype, int32_t ignore_index,
                     float* row_max, float* row_sumexp, float* row_target_logit, void* workspace,
                     size_t workspace_bytes, int64_t chunk_rows, void* stream) {
  if (!valid_dtype(dtype)) return FLCE_E_INVALID_ARG;
  if (N < 0 || H <= 0 || V_local <= 0 || vocab_start < 0 || V_global < vocab_start + V_local ||
      chunk_rows < 0)
    return FLCE_E_INVALID_ARG;
  if (W_shard == nullptr) return FLCE_E_INVALID_ARG;
  if (N > 0 && (X == nullptr || targets == nullptr || row_max == nullptr || row_sumexp == nullptr ||
                row_target_logit == nullptr))
    return FLCE_E_INVALID_ARG;
  if (N >= kMaxRows || H >= kMaxDim || V_global >= kMaxDim) return FLCE_E_UNSUPPORTED;
  const void* ptrs[] = {X, W_shard, bias_shard, targets, row_max, row_sumexp, row_target_logit, workspace};
  for (const void* q : ptrs)
    if (q != nullptr && !aligned16(q)) return FLCE_E_UNSUPPORTED;
  if (is16(dtype) && (H % 8) != 0) return FLCE_E_UNSUPPORTED;
  if (!gemm16_fits(dtype, H, V_local)) return FLCE_E_UNSUPPORTED;
  Plan p;
  if (!make_plan(N, H, V_local, dtype, chunk_rows, &p)) return FLCE_E_INVALID_ARG;
  if (workspace == nullptr || workspace_bytes < p.total) return FLCE_E_WORKSPACE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  WsHeader* hdr = reinterpret_cast<WsHeader*>(ws);
  void* zbuf = ws + p.off_chunk;
  const size_t e = elem_bytes(dtype);
  auto gemm = [dtype](const GemmDesc& d, hipStream_t st) { return gemm_for(dtype, d, st); };
  LCE_TRY(timed(kKindOther, s, [&] {
    return launch_count_targets(targets, N, V_global, ignore_index, FLCE_REDUCTION_SUM, hdr, s);
  }));
  for (int64_t r0 = 0; r0 < N; r0 += p.chunk) {
    const int64_t rows = std::min(p.chunk, N - r0);
    GemmDesc g1{};
    g1.A = static_cast<const char*>(X) + static_cast<size_t>(r0) * H * e;
    g1.lda = H; g1.a_kmajor = true;
    g1.B = W_shard; g1.ldb = H; g1.b_kmajor = true;
    g1.C = zbuf; g1.ldc = p.ldz; g1.bias = bias_shard;
    g1.M = rows; g1.N = V_local; g1.K = H;
    g1.epilogue = kEpiLogits; g1.k_splits = 1;
    LCE_TRY(timed(kKindLogits, s, [&] { return gemm(g1, s); }));
    LCE_TRY(timed(kKindRowCE, s, [&] {
      return launch_shard_stats(dtype, zbuf, p.ldz, rows, V_local, vocab_start, V_global,
                                targets + r0, ignore_index, row_max + r0, row_sumexp + r0,
                                row_target_logit + r0, s);
    }));
  }
  return FLCE_OK;
}

int ce_combine_shard_stats(const float* shard_max, const float* shard_sumexp,
                           const float* shard_target_logit, int64_t P, int64_t N,
                           const int32_t* targets, int64_t V_global, int32_t ignore_index,
                           int reduction, float* row_lse, float* loss, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (reduction < FLCE_REDUCTION_NONE || reduction > FLCE_REDUCTION_MEAN) return FLCE_E_INVALID_ARG;
  if (P <= 0 || N < 0 || V_global <= 0 || loss == nullptr) return FLCE_E_INVALID_ARG;
  if (N > 0 && (shard_max == nullptr || shard_sumexp == nullptr || shard_target_logit == nullptr ||
                targets == nullptr))
    return FLCE_E_INVALID_ARG;
  if (N >= kMaxRows || V_global >= kMaxDim || P >= kMaxDim) return FLCE_E_UNSUPPORTED;
  const void* ptrs[] = {shard_max, shard_sumexp, shard_target_logit, targets, row_lse, loss, workspace};
  for (const void* q : ptrs)
    if (q != nullptr && !aligned16(q)) return FLCE_E_UNSUPPORTED;
  if (workspace == nullptr || workspace_bytes < ce_ws_bytes(N)) return FLCE_E_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  WsHeader* hdr = reinterpret_cast<WsHeader*>(ws);
  float* loss_rows = reduction == FLCE_REDUCTION_NONE ? loss : reinterpret_cast<float*>(ws + align_up(sizeof(WsHeader)));
  LCE_TRY(timed(kKindOther, s, [&] {
    return launch_count_targets(targets, N, V_global, ignore_index, reduction, hdr, s);
  }));
  LCE_TRY(timed(kKindOther, s, [&] {
    return launch_combine_stats(shard_max, shard_sumexp, shard_target_logit, P, N, targets,
                                ignore_index, V_global, row_lse, loss_rows, s);
  }));
  if (reduction != FLCE_REDUCTION_NONE)
    LCE_TRY(timed(kKindOther, s, [&] {
      return launch_reduce_loss(loss_rows, N, hdr, reduction, loss, s);
    }));
  return FLCE_OK;
}

static int shard_backward_impl(const void* X, const void* W_shard, const void* bias_shard,
                               const int32_t* targets, int64_t N, int64_t H, int64_t V_local,
                               int64_t vocab_start, int64_t V_global, int dtype,
                               int32_t ignore_index, int reduction, const float* row_lse,
                               int grad_dtype, void* grad_X, void* grad_W_shard,
                               void* grad_bias_shard, void* workspace, size_t workspace_bytes,
                               int64_t chunk_rows, void* stream) {
  int st = validate_common(dtype, reduction);
  if (st != FLCE_OK) return st;
  if (grad_dtype != FLCE_F32 && grad_dtype != dtype) return FLCE_E_INVALID_ARG;
  const bool g16 = grad_dtype != FLCE_F32;
  const size_t ge = g16 ? 2 : 4;
  if (N < 0 || H <= 0 || V_local <= 0 || vocab_start < 0 || V_global < vocab_start + V_local ||
      chunk_rows < 0)
    return FLCE_E_INVALID_ARG;
  if (W_shard == nullptr) return FLCE_E_INVALID_ARG;
  if (N > 0 && (X == nullptr || targets == nullptr || row_lse == nullptr)) return FLCE_E_INVALID_ARG;
  if (grad_bias_shard != nullptr && bias_shard == nullptr) return FLCE_E_INVALID_ARG;
  if (N >= kMaxRows || H >= kMaxDim || V_global >= kMaxDim) return FLCE_E_UNSUPPORTED;
  const void* ptrs[] = {X, W_shard, bias_shard, targets, row_lse, grad_X, grad_W_shard,
                        grad_bias_shard, workspace};
  for (const void* q : ptrs)
    if (q != nullptr && !aligned16(q)) return FLCE_E_UNSUPPORTED;
  if (is16(dtype) && (H % 8) != 0) return FLCE_E_UNSUPPORTED;
  if (!gemm16_fits(dtype, H, V_local)) return FLCE_E_UNSUPPORTED;
  Plan p;
  if (!make_plan(N, H, V_local, dtype, chunk_rows, &p)) return FLCE_E_INVALID_ARG;
  if (workspace == nullptr || workspace_bytes < p.total) return FLCE_E_WORKSPACE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  WsHeader* hdr = reinterpret_cast<WsHeader*>(ws);
  void* zbuf = ws + p.off_chunk;
  const size_t e = elem_bytes(dtype);
  auto gemm = [dtype](const GemmDesc& d, hipStream_t st) { return gemm_for(dtype, d, st); };
  const GradScaling gsc = grad_scaling(dtype, hdr);

  // Validity and the mean's N_valid are judged against the whole vocabulary.
  LCE_TRY(timed(kKindOther, s, [&] {
    return launch_count_targets(targets, N, V_global, ignore_index, reduction, hdr, s);
  }));
  if (N == 0) {
    if (grad_W_shard)
      LCE_TRY(timed(kKindOther, s, [&] { return launch_zero(grad_W_shard, V_local * H, grad_dtype, s); }));
    if (grad_bias_shard)
      LCE_TRY(timed(kKindOther, s, [&] { return launch_zero(grad_bias_shard, V_local, grad_dtype, s); }));
  }
  // Rows with an ignored or invalid target have zero dlogits over every
  // shard: packed as in flce_chunks (validity against V_global).
  Packer pkr;
  st = pkr.setup(p, ws, hdr, targets, N, V_global, ignore_index, nullptr, grad_X,
                 H * static_cast<int64_t>(ge), s);
  if (st != FLCE_OK) return st;
  for (int64_t r0 = 0; r0 < N; r0 += p.chunk) {
    const int64_t rows = std::min(p.chunk, N - r0);
    const bool first = r0 == 0;
    const RowPack pk = pkr.chunk(r0);
    const char *Xc, *Xt;
    st = pkr.rows_of(X, r0, rows, H, e, s, &Xc, grad_W_shard ? &Xt : nullptr);
    if (st != FLCE_OK) return st;
    if (!grad_W_shard) Xt = nullptr;

    GemmDesc g1{};
    g1.A = Xc; g1.lda = H; g1.a_kmajor = true;
    g1.B = W_shard; g1.ldb = H; g1.b_kmajor = true;
    g1.C = zbuf; g1.ldc = p.ldz; g1.bias = bias_shard;
    g1.M = rows; g1.N = V_local; g1.K = H;
    g1.epilogue = kEpiLogits; g1.k_splits = 1;
    pkr.limit(g1, 0, r0);
    LCE_TRY(timed(kKindLogits, s, [&] { return gemm(g1, s); }));
    LCE_TRY(timed(kKindRowCE, s, [&] {
      return launch_shard_grad(dtype, zbuf, p.ldz, rows, V_local, p.ldz - V_local, vocab_start,
                               V_global, (pkr.on ? pkr.ptgt : targets) + r0, ignore_index,
                               pkr.on ? row_lse : row_lse + r0, hdr, gsc.row_shift, s, pk);
    }));
    if (grad_bias_shard)
      LCE_TRY(timed(kKindOther, s, [&] {
        return launch_colsum(dtype, zbuf, p.ldz, rows, V_local, grad_bias_shard, grad_dtype, !first,
                             gsc.out_scale, gsc.out_shift, s, pk);
      }));
    st = gradient_products(p, dtype, W_shard, H, V_local, zbuf, Xc, Xt, rows, r0, N, first, pkr,
                           pk, grad_X, false, grad_W_shard, grad_dtype, gsc, ws, s);
    if (st != FLCE_OK) return st;
  }
  return FLCE_OK;
}

int flce_shard_backward(const void* X, const void* W_shard, const void* bias_shard,
                        const int32_t* targets, int64_t N, int64_t H, int64_t V_local,
                        int64_t vocab_start, int64_t V_global, int dtype, int32_t ignore_index,
                        int reduction, const float* row_lse, float* grad_X, float* grad_W_shard,
                        float* grad_bias_shard, void* workspace, size_t workspace_bytes,
                        int64_t chunk_rows, void* stream) {
  return shard_backward_impl(X, W_shard, bias_shard, targets, N, H, V_local, vocab_start, V_global,
                             dtype, ignore_index, reduction, row_lse, FLCE_F32, grad_X,
                             grad_W_shard, grad_bias_shard, workspace, workspace_bytes, chunk_rows,
                             stream);
}

int flce_shard_backward_ex(const void* X, const void* W_shard, const void* bias_shard,
                           const int32_t* targets, int64_t N, int64_t H, int64_t V_local,
                           int64_t vocab_start, int64_t V_global, int dtype, int32_t ignore_index,
                           int reduction, const float* row_lse, int grad_dtype, void* grad_X,
                           void* grad_W_shard, void* grad_bias_shard, void* workspace,
                           size_t workspace_bytes, int64_t chunk_rows, void* stream) {
  return shard_backward_impl(X, W_shard, bias_shard, targets, N, H, V_local, vocab_start, V_global,
                             dtype, ignore_index, reduction, row_lse, grad_dtype, grad_X,
                             grad_W_shard, grad_bias_shard, workspace, workspace_bytes, chunk_rows,
                             stream);
}

size_t flce_jsd_workspace_bytes(int64_t N, int64_t H_s, int64_t V, int dtype, int64_t chunk_rows) {
  Plan p;
  if (!make_plan(N, H_s, V, dtype, chunk_rows, &p)) return 0;
  return p.total + align_up(static_cast<size_t>(p.chunk) * static_cast<size_t>(p.ldz) * elem_bytes(dtype));
}

static int jsd_impl(const void* X_s, const void* W_s, const void* X_t, const void* W_t,
                    const int32_t* targets, int64_t N, int64_t H_s, int64_t H_t, int64_t V,
                    int dtype, int32_t ignore_index, int reduction, float temperature,
                    int grad_dtype, float* loss, void* grad_X_s, void* grad_W_s, void* workspace,
                    size_t workspace_bytes, int64_t chunk_rows, void* stream) {
  int st = validate_flce(X_s, W_s, nullptr, targets, N, H_s, V, dtype, reduction, loss, grad_X_s,
                         grad_W_s, nullptr, chunk_rows, workspace);
  if (st != FLCE_OK) return st;
  if (grad_dtype != FLCE_F32 && grad_dtype != dtype) return FLCE_E_INVALID_ARG;
  const bool g16 = grad_dtype != FLCE_F32;
  const size_t ge = g16 ? 2 : 4;
  if (W_t == nullptr || H_t <= 0 || !(temperature > 0.0f)) return FLCE_E_INVALID_ARG;
  if (N > 0 && X_t == nullptr) return FLCE_E_INVALID_ARG;
  if (H_t >= kMaxDim) return FLCE_E_UNSUPPORTED;
  if ((X_t != nullptr && !aligned16(X_t)) || !aligned16(W_t)) return FLCE_E_UNSUPPORTED;
  if (is16(dtype) && (H_t % 8) != 0) return FLCE_E_UNSUPPORTED;
  if (!gemm16_fits(dtype, H_t, V)) return FLCE_E_UNSUPPORTED;
  Plan p;
  if (!make_plan(N, H_s, V, dtype, chunk_rows, &p)) return FLCE_E_INVALID_ARG;
  const size_t e = elem_bytes(dtype);
  const size_t tbuf = p.total;  // the teacher's chunk logits follow the FLCE layout
  if (workspace == nullptr ||
      workspace_bytes < tbuf + align_up(static_cast<size_t>(p.chunk) * static_cast<size_t>(p.ldz) * e))
    return FLCE_E_WORKSPACE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  WsHeader* hdr = reinterpret_cast<WsHeader*>(ws);
  float* loss_rows = reduction == FLCE_REDUCTION_NONE ? loss : reinterpret_cast<float*>(ws + p.off_rows);
  void* zs = ws + p.off_chunk;
  void* zt = ws + tbuf;
  float* split_buf = reinterpret_cast<float*>(ws + p.off_split);
  auto gemm = [dtype](const GemmDesc& d, hipStream_t st2) { return gemm_for(dtype, d, st2); };
  const float inv_tau = 1.0f / temperature;
  const GradScaling gsc = grad_scaling(dtype, hdr, inv_tau);

  LCE_TRY(timed(kKindOther, s, [&] {
    return launch_count_targets(targets, N, V, ignore_index, reduction, hdr, s);
  }));
  if (N == 0 && grad_W_s)
    LCE_TRY(timed(kKindOther, s, [&] { return launch_zero(grad_W_s, V * H_s, grad_dtype, s); }));
  // Packed rows (as in flce_chunks) when the teacher's gathered hidden states
  // fit the split-K partial buffer after the student's: the buffer is free
  // from the gather until the grad_X product, and the teacher's rows are read
  // only by the teacher's logits product.
  const size_t split_bytes = p.off_map - p.off_split;
  const size_t xs_bytes = align_up(static_cast<size_t>(p.chunk) * static_cast<size_t>(H_s) * e);
  const bool teacher_fits =
      xs_bytes + static_cast<size_t>(p.chunk) * static_cast<size_t>(H_t) * e <= split_bytes;
  Packer pkr;
  // The teacher's rows take the partial buffer's second half, so the student's
  // grad_W reads its gathered rows as they are (no transposed copy).
  st = pkr.setup(p, ws, hdr, targets, N, V, ignore_index, loss_rows, grad_X_s,
                 H_s * static_cast<int64_t>(ge), s, teacher_fits, false);
  if (st != FLCE_OK) return st;
  for (int64_t r0 = 0; r0 < N; r0 += p.chunk) {
    const int64_t rows = std::min(p.chunk, N - r0);
    const bool first = r0 == 0;
    const RowPack pk = pkr.chunk(r0);
    const char* Xs_c;
    st = pkr.rows_of(X_s, r0, rows, H_s, e, s, &Xs_c);
    if (st != FLCE_OK) return st;
    const char* Xt_c = static_cast<const char*>(X_t) + static_cast<size_t>(r0) * H_t * e;
    if (pkr.on) {
      LCE_TRY(timed(kKindOther, s, [&] {
        return launch_gather_rows(X_t, H_t * static_cast<int64_t>(e), rows, pk,
                                  reinterpret_cast<char*>(split_buf) + xs_bytes, s);
      }));
      Xt_c = reinterpret_cast<const char*>(split_buf) + xs_bytes;
    }
    GemmDesc gs{};
    gs.A = Xs_c; gs.lda = H_s; gs.a_kmajor = true;
    gs.B = W_s; gs.ldb = H_s; gs.b_kmajor = true;
    gs.C = zs; gs.ldc = p.ldz; gs.M = rows; gs.N = V; gs.K = H_s;
    gs.epilogue = kEpiLogits; gs.k_splits = 1;
    pkr.limit(gs, 0, r0);
    LCE_TRY(timed(kKindLogits, s, [&] { return gemm(gs, s); }));
    GemmDesc gt = gs;
    gt.A = Xt_c; gt.lda = H_t; gt.B = W_t; gt.ldb = H_t; gt.C = zt; gt.K = H_t;
    LCE_TRY(timed(kKindLogits, s, [&] { return gemm(gt, s); }));
    LCE_TRY(timed(kKindRowCE, s, [&] {
      return launch_row_jsd(dtype, zs, zt, p.ldz, rows, V, p.ldz - V, inv_tau,
                            (pkr.on ? pkr.ptgt : targets) + r0, ignore_index, hdr,
                            pkr.on ? loss_rows : loss_rows + r0, gsc.row_shift, s, pk);
    }));
    st = gradient_products(p, dtype, W_s, H_s, V, zs, Xs_c, nullptr, rows, r0, N, first, pkr, pk, grad_X_s,
                           false, grad_W_s, grad_dtype, gsc, ws, s);
    if (st != FLCE_OK) return st;
  }
  if (reduction != FLCE_REDUCTION_NONE)
    LCE_TRY(timed(kKindOther, s, [&] {
      return launch_reduce_loss(loss_rows, N, hdr, reduction, loss, s);
    }));
  return FLCE_OK;
}

int flce_jsd_forward_backward(const void* X_s, const void* W_s, const void* X_t, const void* W_t,
                              const int32_t* targets, int64_t N, int64_t H_s, int64_t H_t,
                              int64_t V, int dtype, int32_t ignore_index, int reduction,
                              float temperature, float* loss, float* grad_X_s, float* grad_W_s,
                              void* workspace, size_t workspace_bytes, int64_t chunk_rows,
                              void* stream) {
  return jsd_impl(X_s, W_s, X_t, W_t, targets, N, H_s, H_t, V, dtype, ignore_index, reduction,
                  temperature, FLCE_F32, loss, grad_X_s, grad_W_s, workspace, workspace_bytes,
                  chunk_rows, stream);
}

int flce_jsd_forward_backward_ex(const void* X_s, const void* W_s, const void* X_t, const void* W_t,
                                 const int32_t* targets, int64_t N, int64_t H_s, int64_t H_t,
                                 int64_t V, int dtype, int32_t ignore_index, int reduction,
                                 float temperature, int grad_dtype, float* loss, void* grad_X_s,
                                 void* grad_W_s, void* workspace, size_t workspace_bytes,
                                 int64_t chunk_rows, void* stream) {
  return jsd_impl(X_s, W_s, X_t, W_t, targets, N, H_s, H_t, V, dtype, ignore_index, reduction,
                  temperature, grad_dtype, loss, grad_X_s, grad_W_s, workspace, workspace_bytes,
                  chunk_rows, stream);
}

size_t flce_dpo_workspace_bytes(int64_t n_pairs, int64_t seq_len, int64_t H, int64_t V, int dtype,
                                int64_t chunk_rows) {
  if (n_pairs < 0 || seq_len <= 0 || n_pairs * seq_len >= kMaxRows) return 0;
  const int64_t N = 2 * n_pairs * seq_len;
  Plan p;
  if (!make_plan(N, H, V, dtype, chunk_rows, &p)) return 0;
  return p.total + align_up(static_cast<size_t>(std::max<int64_t>(N, 1)) * sizeof(float)) +
         align_up(static_cast<size_t>(std::max<int64_t>(2 * n_pairs, 1)) * sizeof(double));
}

static int dpo_impl(const void* X, const void* W, const int32_t* targets, int64_t n_pairs,
                    int64_t seq_len, int64_t H, int64_t V, int dtype, int32_t ignore_index,
                    const float* ref_logps, float beta, int grad_dtype, float* loss,
                    float* pair_loss, void* grad_X, void* grad_W, void* workspace,
                    size_t workspace_bytes, int64_t chunk_rows, void* stream) {
  if (n_pairs < 0 || seq_len <= 0 || n_pairs * seq_len >= kMaxRows) return FLCE_E_INVALID_ARG;
  if (grad_dtype != FLCE_F32 && grad_dtype != dtype) return FLCE_E_INVALID_ARG;
  const bool g16 = grad_dtype != FLCE_F32;
  const size_t ge = g16 ? 2 : 4;
  if (!(beta > 0.0f)) return FLCE_E_INVALID_ARG;
  const int64_t N = 2 * n_pairs * seq_len;
  int st = validate_flce(X, W, nullptr, targets, N, H, V, dtype, FLCE_REDUCTION_SUM, loss, grad_X,
                         grad_W, nullptr, chunk_rows, workspace);
  if (st != FLCE_OK) return st;
  if (n_pairs > 0 && ref_logps == nullptr) return FLCE_E_INVALID_ARG;
  if ((ref_logps != nullptr && !aligned16(ref_logps)) || (pair_loss != nullptr && !aligned16(pair_loss)))
    return FLCE_E_UNSUPPORTED;
  Plan p;
  if (!make_plan(N, H, V, dtype, chunk_rows, &p)) return FLCE_E_INVALID_ARG;
  const size_t off_scale = p.total;
  const size_t off_logp = off_scale + align_up(static_cast<size_t>(std::max<int64_t>(N, 1)) * sizeof(float));
  if (workspace == nullptr ||
      workspace_bytes < off_logp + align_up(static_cast<size_t>(std::max<int64_t>(2 * n_pairs, 1)) * sizeof(double)))
    return FLCE_E_WORKSPACE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  WsHeader* hdr = reinterpret_cast<WsHeader*>(ws);
  float* loss_rows = reinterpret_cast<float*>(ws + p.off_rows);
  float* row_scale = reinterpret_cast<float*>(ws + off_scale);
  double* logp = reinterpret_cast<double*>(ws + off_logp);
  void* zbuf = ws + p.off_chunk;
  const size_t e = elem_bytes(dtype);
  auto gemm = [dtype](const GemmDesc& d, hipStream_t st2) { return gemm_for(dtype, d, st2); };
  // Rows with an ignored or invalid target (the masked prompt tokens) add
  // nothing to the log-probabilities or the gradients: both passes run over
  // the packed rows (as in flce_chunks).
  Packer pkr;
  // Chunk rows (gathered when packed; transposed too when grad_W is wanted,
  // also in the first pass, whose rows the second reuses for a single chunk)
  // and their logits.
  auto logits = [&](int64_t r0, int64_t rows, const char** Xc, const char** Xt) {
    int r = pkr.rows_of(X, r0, rows, H, e, s, Xc, grad_W ? Xt : nullptr);
    if (!grad_W) *Xt = nullptr;
    if (r != FLCE_OK) return hipErrorUnknown;
    GemmDesc g1{};
    g1.A = *Xc;
    g1.lda = H; g1.a_kmajor = true;
    g1.B = W; g1.ldb = H; g1.b_kmajor = true;
    g1.C = zbuf; g1.ldc = p.ldz; g1.M = rows; g1.N = V; g1.K = H;
    g1.epilogue = kEpiLogits; g1.k_splits = 1;
    pkr.limit(g1, 0, r0);
    return timed(kKindLogits, s, [&] { return gemm(g1, s); });
  };

  // Validity of every target row (the scale itself is unused: the factors
  // come per row from the pairs).
  LCE_TRY(timed(kKindOther, s, [&] {
    return launch_count_targets(targets, N, V, ignore_index, FLCE_REDUCTION_SUM, hdr, s);
  }));
  if (N == 0 && grad_W)
    LCE_TRY(timed(kKindOther, s, [&] { return launch_zero(grad_W, V * H, grad_dtype, s); }));
  st = pkr.setup(p, ws, hdr, targets, N, V, ignore_index, loss_rows, grad_X,
                 H * static_cast<int64_t>(ge), s);
  if (st != FLCE_OK) return st;
  const int32_t* tg = pkr.on ? pkr.ptgt : targets;
  // Pass 1: the CE row losses of every row (= minus the token log-probabilities).
  const char* Xc = nullptr;
  const char* Xt = nullptr;
  for (int64_t r0 = 0; r0 < N; r0 += p.chunk) {
    const int64_t rows = std::min(p.chunk, N - r0);
    LCE_TRY(logits(r0, rows, &Xc, &Xt));
    LCE_TRY(timed(kKindRowCE, s, [&] {
      return launch_row_ce(dtype, zbuf, p.ldz, nullptr, p.ldz, rows, V, p.ldz - V, tg + r0,
                           ignore_index, hdr, pkr.on ? loss_rows : loss_rows + r0, nullptr, 0, s,
                           pkr.chunk(r0));
    }));
  }
  LCE_TRY(timed(kKindOther, s, [&] {
    return launch_dpo(loss_rows, n_pairs, seq_len, ref_logps, beta, logp, loss, pair_loss,
                      row_scale, s);
  }));
  // Pass 2: per-row weighted dlogits and the two gradient products. With a
  // single chunk its logits (and gathered rows) are still in the buffers
  // (pass 1 only read them).
  const bool one_chunk = N <= p.chunk;
  // The rows carry their own factors, |±beta sigma(-d) / P| <= beta / P.
  const GradScaling gsc =
      grad_scaling(dtype, nullptr, static_cast<double>(beta) / static_cast<double>(std::max<int64_t>(n_pairs, 1)));
  for (int64_t r0 = 0; r0 < N && (grad_X || grad_W); r0 += p.chunk) {
    const int64_t rows = std::min(p.chunk, N - r0);
    const bool first = r0 == 0;
    const RowPack pk = pkr.chunk(r0);
    if (!one_chunk) LCE_TRY(logits(r0, rows, &Xc, &Xt));
    LCE_TRY(timed(kKindRowCE, s, [&] {
      return launch_row_ce(dtype, zbuf, p.ldz, zbuf, p.ldz, rows, V, p.ldz - V, tg + r0,
                           ignore_index, hdr, pkr.on ? loss_rows : loss_rows + r0,
                           pkr.on ? row_scale : row_scale + r0, gsc.row_shift, s, pk);
    }));
    st = gradient_products(p, dtype, W, H, V, zbuf, Xc, Xt, rows, r0, N, first, pkr, pk, grad_X, false,
                           grad_W, grad_dtype, gsc, ws, s);
    if (st != FLCE_OK) return st;
  }
  return FLCE_OK;
}

int flce_dpo_forward_backward(const void* X, const void* W, const int32_t* targets, int64_t n_pairs,
                              int64_t seq_len, int64_t H, int64_t V, int dtype,
                              int32_t ignore_index, const float* ref_logps, float beta,
                              float* loss, float* pair_loss, float* grad_X, float* grad_W,
                              void* workspace, size_t workspace_bytes, int64_t chunk_rows,
                              void* stream) {
  return dpo_impl(X, W, targets, n_pairs, seq_len, H, V, dtype, ignore_index, ref_logps, beta,
                  FLCE_F32, loss, pair_loss, grad_X, grad_W, workspace, workspace_bytes,
                  chunk_rows, stream);
}

int flce_dpo_forward_backward_ex(const void* X, const void* W, const int32_t* targets,
                                 int64_t n_pairs, int64_t seq_len, int64_t H, int64_t V, int dtype,
                                 int32_t ignore_index, const float* ref_logps, float beta,
                                 int grad_dtype, float* loss, float* pair_loss, void* grad_X,
                                 void* grad_W, void* workspace, size_t workspace_bytes,
                                 int64_t chunk_rows, void* stream) {
  return dpo_impl(X, W, targets, n_pairs, seq_len, H, V, dtype, ignore_index, ref_logps, beta,
                  grad_dtype, loss, pair_loss, grad_X, grad_W, workspace, workspace_bytes,
                  chunk_rows, stream);
}

int flce_shift_labels(const int32_t* labels, int64_t B, int64_t S, int32_t ignore_index,
                      int32_t* targets, void* stream) {
  if (B < 0 || S <= 0) return FLCE_E_INVALID_ARG;
  if (B > 0 && (labels == nullptr || targets == nullptr)) return FLCE_E_INVALID_ARG;
  if (B * S >= kMaxRows || B >= kMaxRows) return FLCE_E_UNSUPPORTED;
  if (B > 0 && labels == targets) return FLCE_E_INVALID_ARG;  // not in place
  hipStream_t s = static_cast<hipStream_t>(stream);
  LCE_TRY(timed(kKindOther, s, [&] { return launch_shift_labels(labels, B, S, ignore_index, targets, s); }));
  return FLCE_OK;
}

int flce_check_device_error(const void* workspace, void* stream) {
  if (workspace == nullptr) return FLCE_E_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipStreamSynchronize(s) != hipSuccess) return FLCE_E_HIP;
  int32_t n_bad = 0;
  if (hipMemcpy(&n_bad, workspace, sizeof(n_bad), hipMemcpyDeviceToHost) != hipSuccess) return FLCE_E_HIP;
  return n_bad != 0 ? FLCE_E_TARGET : FLCE_OK;
}

int flce_timing_enable(int enable) {
  g_timing = enable != 0;
  return FLCE_OK;
}

int flce_timing_read(int kind, double* total_ms, int64_t* launches) {
  double ms = 0.0;
  int64_t count = 0;
  for (const TimedLaunch& r : g_records) {
    if (r.kind != kind) continue;
    if (hipEventSynchronize(r.stop) != hipSuccess) return FLCE_E_HIP;
    float t = 0.0f;
    if (hipEventElapsedTime(&t, r.start, r.stop) != hipSuccess) return FLCE_E_HIP;
    ms += t;
    ++count;
  }
  if (total_ms) *total_ms = ms;
  if (launches) *launches = count;
  return FLCE_OK;
}

int flce_timing_reset(void) {
  for (const TimedLaunch& r : g_records) {
    if (hipEventSynchronize(r.stop) != hipSuccess) return FLCE_E_HIP;
    g_event_pool.push_back(r.start);
    g_event_pool.push_back(r.stop);
  }
  g_records.clear();
  return FLCE_OK;
}

}  // extern "C"
