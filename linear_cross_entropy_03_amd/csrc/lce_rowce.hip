// Row kernels of the FLCE / CE path (HBM-bound, no MFMA):
//   * target counting (valid rows, bad targets, reduction scale),
//   * the fused row cross-entropy: logsumexp, target logit, loss and the
//     in-place softmax-minus-one-hot gradient (liger-kernel README, "Kernels":
//     CrossEntropy computes loss and gradient in one pass and may replace the
//     input logits with the gradient; torchtune + Liger blog, Figure 1 text:
//     each chunk's loss and logits gradient come from that CE kernel),
//   * per-shard statistics (DeepSpeed vocab-parallel CE page),
//   * the deterministic loss reduction, bias-gradient column sums, split-K
//     reduction and a fill kernel.
//
// One workgroup owns one row. Rows are streamed with 16-byte loads; when a row
// fits in the workgroup's registers (up to 16 vectors per lane) it is read
// from HBM once and the gradient is computed from the registers, so the row
// costs one read and one write.
#include "lce_common.h"

namespace lce {

// ------------------------------------------------------------ target count

__global__ __launch_bounds__(1024) void k_count_targets(const int32_t* __restrict__ t, int64_t n,
                                                        int64_t V, int32_t ign, int reduction,
                                                        WsHeader* __restrict__ hdr) {
  __shared__ int s_valid, s_bad;
  if (threadIdx.x == 0) { s_valid = 0; s_bad = 0; }
  __syncthreads();
  int valid = 0, bad = 0;
  auto count = [&](int32_t y) {
    if (y == ign) return;
    if (y >= 0 && static_cast<int64_t>(y) < V) ++valid; else ++bad;
  };
  // 16-byte loads, several in flight per lane, then the unaligned rest.
  const int64_t n4 = (reinterpret_cast<uintptr_t>(t) & 15u) == 0 ? n / 4 : 0;
  const int4* t4 = reinterpret_cast<const int4*>(t);
#pragma unroll 8
  for (int64_t i = threadIdx.x; i < n4; i += 1024) {
    const int4 v = t4[i];
    count(v.x); count(v.y); count(v.z); count(v.w);
  }
  for (int64_t i = n4 * 4 + threadIdx.x; i < n; i += 1024) count(t[i]);
  atomicAdd(&s_valid, valid);  // integer sums: exact in any order
  atomicAdd(&s_bad, bad);
  __syncthreads();
  if (threadIdx.x == 0) {
    hdr->n_bad = s_bad;
    hdr->n_valid = s_valid;
    // reduction: 0 none, 1 sum, 2 mean
    hdr->scale = (reduction == 2) ? (s_valid > 0 ? 1.0f / static_cast<float>(s_valid) : 0.0f) : 1.0f;
  }
}

hipError_t launch_count_targets(const int32_t* targets, int64_t n, int64_t V, int32_t ignore_index,
                                int reduction, WsHeader* hdr, hipStream_t s) {
  hipLaunchKernelGGL(k_count_targets, dim3(1), dim3(1024), 0, s, targets, n, V, ignore_index,
                     reduction, hdr);
  return hipGetLastError();
}

// ------------------------------------------------------------------ row CE

// Row geometry: `head` scalar elements up to 16-byte alignment, `nvec`
// 16-byte vectors, then the scalar tail [tail0, V).
struct RowSplit {
  int64_t head, nvec, tail0;
};
template <typename T>
__device__ __forceinline__ RowSplit split_row(const T* z, int64_t V) {
  constexpr int kVec = Elem<T>::kVec;
  const uintptr_t a = reinterpret_cast<uintptr_t>(z);
  int64_t head = static_cast<int64_t>(((16u - (a & 15u)) & 15u) / sizeof(T));
  if (head > V) head = V;
  const int64_t nvec = (V - head) / kVec;
  return {head, nvec, head + nvec * kVec};
}

// Fold x into a running (max, sum of exp(x - max)) pair.
__device__ __forceinline__ void online_push(float& m, float& s, float x) {
  const float mn = fmaxf(m, x);
  s = s * __builtin_amdgcn_exp2f((m - mn) * kLog2e) + __builtin_amdgcn_exp2f((x - mn) * kLog2e);
  m = mn;
}
template <int kN>
__device__ __forceinline__ void online_push_vec(float& m, float& s, const float* f) {
  float vm = f[0];
#pragma unroll
  for (int i = 1; i < kN; ++i) vm = fmaxf(vm, f[i]);
  const float mn = fmaxf(m, vm);
  float acc = s * __builtin_amdgcn_exp2f((m - mn) * kLog2e);
#pragma unroll
  for (int i = 0; i < kN; ++i) acc += __builtin_amdgcn_exp2f((f[i] - mn) * kLog2e);
  s = acc;
  m = mn;
}

// Block-wide (max, sumexp) from per-lane online pairs.
template <int kThreads>
__device__ __forceinline__ void block_lse_parts(float m, float s, float* red0, float* red1,
                                                float& M, float& S) {
  M = block_max<kThreads>(m, red0);
  const float mine = (m == -INFINITY) ? 0.0f : s * __builtin_amdgcn_exp2f((m - M) * kLog2e);
  S = block_sum<kThreads>(mine, red1);
}

// The sum pass of the register-resident row kernels in base 2, one fma per
// element: a lane with maximum m sums 2^(x log2e - m2), m2 = m log2e rounded
// to float. Rounding is monotone, so the row's largest m2 is M log2e rounded
// (M the row maximum), and 2^(x log2e - M2) = e^(x - M) 2^eps with
// eps = M log2e - M2, which an fma gives exactly; the row's
// lse = M + (log2 S - eps) ln 2 keeps M exact. No contraction here: m2 and
// M2 must be the same rounded products the lanes used.
__device__ __forceinline__ float lane_m2(float m) {
#pragma clang fp contract(off)
  return m * kLog2e;
}
__device__ __forceinline__ float lane_m2_by(float m, float k) {
#pragma clang fp contract(off)
  return m * k;
}
template <int kThreads>
__device__ __forceinline__ float block_lse2(float m, float s, float* red0, float* red1) {
#pragma clang fp contract(off)
  const float M = block_max<kThreads>(m, red0);
  const float M2 = lane_m2(M);
  const float mine = (m == -INFINITY) ? 0.0f : s * __builtin_amdgcn_exp2f(lane_m2(m) - M2);
  const float S = block_sum<kThreads>(mine, red1);
  const float eps = fmaf(M, kLog2e, -M2);
  return M + (__builtin_amdgcn_logf(S) - eps) * kLn2;
}

// Gradient of one 16-byte vector of a row with a valid target:
// c exp(x - lse) per element, and gt = c (exp(x_t - lse) - 1), computed once
// per row from the target logit x_t, for the target when it falls in this
// vector (rel = target - the vector's first column, in [0, kVec); |rel| <
// 2^30 since V < 2^30). Only the target's lane takes that branch, once per
// row, so the other elements carry no per-element compare.
template <typename T>
__device__ __forceinline__ uint4 ce_grad_vec(const uint4& v, int rel, float c, float lse, float gt) {
  using E = Elem<T>;
  constexpr int kVec = E::kVec;
  float f[kVec];
  E::unpack(v, f);
#pragma unroll
  for (int i = 0; i < kVec; ++i) f[i] = c * __builtin_amdgcn_exp2f((f[i] - lse) * kLog2e);
  if (static_cast<unsigned>(rel) < static_cast<unsigned>(kVec)) {
    asm volatile("");  // a branch, not per-element selects
#pragma unroll
    for (int i = 0; i < kVec; ++i)
      if (i == rel) f[i] = gt;
  }
  return E::pack(f);
}

// Target count inside the row kernel, for calls of one launch over few rows:
// every workgroup counts all n targets itself (n * 4 bytes from L2) and
// workgroup 0 writes the header, which saves the separate count launch.
struct SelfCount {
  int64_t n;        // rows of the call; 0: read the scale from the header
  int reduction;    // 0 none, 1 sum, 2 mean
  WsHeader* out;    // header written by workgroup 0
  int nt_grad;      // gradient stores non-temporal (the caller's gradient is not reread here)
};

// The reduction's gradient factor from all targets of the call (same rules
// as k_count_targets).
// Raw buffer descriptor over [base, base + bytes) (bytes < 2^31) in scalar
// registers: loads outside the range return zero, so loads need no branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* base, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(a)));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(a >> 32)));
  const int n = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo),
                                           static_cast<short>(0), n, 0x00020000);
}

// Vectors per lane in flight in a streaming pass over a row too long for
// registers.
constexpr int kStream = 8;
// The batched passes address the row through 32-bit buffer offsets,
// including the last batch's lanes past its end.
__device__ __forceinline__ bool stream_batched(int64_t nvec, int threads) {
  return (nvec + static_cast<int64_t>(kStream) * threads) * 16 < (int64_t(1) << 31);
}

// f(vi, v) for every 16-byte vector vi < nvec of one row (zv), lane-strided
// (vector j kThreads + tid of each batch goes to lane tid): kStream
// range-checked loads per lane in flight before any is used. f may write
// vector vi in place (it was loaded by the same lane). kRev walks the
// batches from the row's end: a pass right after a forward pass over the
// same row then starts on the bytes fetched last, the likeliest to be still
// in the L2 and the last-level cache.
template <int kThreads, bool kRev = false, typename F>
__device__ __forceinline__ void stream_row(const uint4* zv, int64_t nvec, F&& f) {
  const int tid = threadIdx.x;
  const int64_t nbatch = stream_batched(nvec, kThreads) ? nvec : 0;
  for (int64_t vi = nbatch + tid; vi < nvec; vi += kThreads) f(vi, zv[vi]);
  if (nbatch == 0) return;
  const __amdgpu_buffer_rsrc_t rv = row_rsrc(zv, nvec * 16);
  constexpr int64_t kBatch = static_cast<int64_t>(kStream) * kThreads;
  const int64_t last = (nbatch - 1) / kBatch * kBatch;
  for (int64_t i = 0; i <= last; i += kBatch) {
    const int64_t b0 = kRev ? last - i : i;
    uint4 sb[kStream];
#pragma unroll
    for (int j = 0; j < kStream; ++j)
      sb[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                            rv, static_cast<int>((b0 + j * kThreads + tid) * 16), 0, 0));
#pragma unroll
    for (int j = 0; j < kStream; ++j) {
      const int64_t vi = b0 + j * kThreads + tid;
      if (vi < nvec) f(vi, sb[j]);
    }
  }
}

// One element's bits through a buffer descriptor (zero out of range).
template <typename T>
__device__ __forceinline__ T load_elem_bits(__amdgpu_buffer_rsrc_t r, int voff) {
  if constexpr (sizeof(T) == 2)
    return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b16(r, voff, 0, 0));
  else
    return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0));
}

// Per-wave target counts into cnt[0][wave] (valid) and cnt[1][wave] (bad);
// read with count_finish after the next barrier. `first` is t[threadIdx.x]
// (ign past the end), loaded by the caller before the row: loads complete in
// order, so a target load issued after the row's would wait for the whole row.
template <int kThreads>
__device__ __forceinline__ void count_partial(const SelfCount& sc, const int32_t* __restrict__ t,
                                              int64_t V, int32_t ign, int32_t first,
                                              float (*cnt)[kThreads / 64]) {
  int valid = 0, bad = 0;
  auto tally = [&](int32_t y) {
    if (y == ign) return;
    if (y >= 0 && static_cast<int64_t>(y) < V) ++valid; else ++bad;
  };
  tally(first);
  for (int64_t i = threadIdx.x + kThreads; i < sc.n; i += kThreads) tally(t[i]);
  // Counts stay below 2^24, so float sums are exact.
  const float v = wave_sum(static_cast<float>(valid)), b = wave_sum(static_cast<float>(bad));
  if ((threadIdx.x & 63) == 0) {
    cnt[0][threadIdx.x >> 6] = v;
    cnt[1][threadIdx.x >> 6] = b;
  }
}

// The reduction's gradient factor from the per-wave counts (same rules as
// k_count_targets); workgroup 0 writes the header.
template <int kThreads>
__device__ __forceinline__ float count_finish(const SelfCount& sc, const float (*cnt)[kThreads / 64]) {
  float v = 0.0f, b = 0.0f;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) {
    v += cnt[0][w];
    b += cnt[1][w];
  }
  const int nv = static_cast<int>(v);
  const float scale = sc.reduction == 2 ? (nv > 0 ? 1.0f / static_cast<float>(nv) : 0.0f) : 1.0f;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    sc.out->n_bad = static_cast<int>(b);
    sc.out->n_valid = nv;
    sc.out->scale = scale;
  }
  return scale;
}

// A 16-byte gradient vector: non-temporal when the caller does not reread it
// here (standalone CE), else a plain store (the FLCE products read the
// chunk's dlogits next).
typedef unsigned u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_grad_vec(uint4* p, const uint4& v, int nt) {
  if (nt) __builtin_nontemporal_store(__builtin_bit_cast(u32x4_nt, v), reinterpret_cast<u32x4_nt*>(p));
  else *p = v;
}

template <typename T, int kThreads, int kRes>
__device__ __forceinline__ void row_ce_grad(const T* Z, int64_t ldz, T* G, int64_t ldg, int64_t V,
                                            int64_t pad_cols, int64_t row, int32_t y, bool valid,
                                            float lse, float zt, const RowSplit& rs, const uint4* buf,
                                            const float* __restrict__ row_scale, int64_t orow,
                                            int grad_shift, float red_scale, int nt);

// kRes > 0: the row's vectors stay in registers (kRes per lane); kRes == 0:
// two streaming passes over the row. Z and G may be the same rows (in-place),
// so neither is declared __restrict__.
template <typename T, int kThreads, int kRes>
__global__ __launch_bounds__(kThreads) void k_row_ce(const T* Z, int64_t ldz, T* G,
                                                     int64_t ldg, int64_t V, int64_t pad_cols,
                                                     const int32_t* __restrict__ targets,
                                                     int32_t ign, const WsHeader* __restrict__ hdr,
                                                     float* __restrict__ loss_rows,
                                                     const float* __restrict__ row_scale,
                                                     int grad_shift, SelfCount sc, RowPack pk) {
  using E = Elem<T>;
  constexpr int kVec = E::kVec;
  __shared__ float red0[kThreads / 64], red1[kThreads / 64];
  __shared__ float cnt[2][kThreads / 64];  // self-count: per-wave target counts
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  // Packed chunks: rows past the live count do not exist (whole workgroup).
  if (pk.live != nullptr && row >= static_cast<int64_t>(*pk.live) - pk.base) return;
  const T* z = Z + row * ldz;
  const int32_t y = targets[row];
  const bool valid = (y != ign) && y >= 0 && static_cast<int64_t>(y) < V;
  const RowSplit rs = split_row(z, V);
  const uint4* zv = reinterpret_cast<const uint4*>(z + rs.head);

  // The target logit (every lane: the gradient needs it) is read before any
  // lane can overwrite the row: the block reductions below end in
  // __syncthreads, which waits for every load of the wave, and all writes
  // come after them. In the register-resident path it is loaded after the
  // row so the row's loads go out first.
  float zt = 0.0f;
  T zt_bits{};
  if (kRes == 0 && valid) zt = E::load(z + y);

  float m = -INFINITY, s = 0.0f, self_scale = 0.0f;
  const int32_t t_first = (sc.n > 0 && tid < sc.n) ? targets[tid] : ign;
  uint4 buf[kRes > 0 ? kRes : 1];
  if constexpr (kRes > 0) {
    // Branch-free loads (zeros past the row's vectors), then the target
    // element (every lane reads the same one; zero when the row is ignored),
    // so the waits below can count loads exactly. Rows here hold at most
    // 16 x kThreads vectors, so byte offsets fit in 32 bits.
    const __amdgpu_buffer_rsrc_t rv = row_rsrc(zv, rs.nvec * 16);
#pragma unroll
    for (int j = 0; j < kRes; ++j)
      buf[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                              rv, (j * kThreads + tid) * 16, 0, 0));
    zt_bits = load_elem_bits<T>(row_rsrc(z, V * static_cast<int64_t>(sizeof(T))),
                                valid ? static_cast<int>(y * sizeof(T)) : 0x7FFFFFF0);
    // The count overlaps the row's loads in flight.
    if (sc.n > 0) count_partial<kThreads>(sc, targets, V, ign, t_first, cnt);
    // max first, then one exp per element against the lane maximum.
    float lm = -INFINITY;
#pragma unroll
    for (int j = 0; j < kRes; ++j) {
      const int64_t vi = static_cast<int64_t>(j) * kThreads + tid;
      if (vi < rs.nvec) {
        float f[kVec];
        E::unpack(buf[j], f);
#pragma unroll
        for (int i = 0; i < kVec; ++i) lm = fmaxf(lm, f[i]);
      }
    }
    if (tid < rs.head) lm = fmaxf(lm, E::load(z + tid));
    if (tid < V - rs.tail0) lm = fmaxf(lm, E::load(z + rs.tail0 + tid));
    // Base-2 sum against the lane maximum (block_lse2).
    float ls = 0.0f;
    if (lm != -INFINITY) {
      const float nm2 = -lane_m2(lm);
#pragma unroll
      for (int j = 0; j < kRes; ++j) {
        const int64_t vi = static_cast<int64_t>(j) * kThreads + tid;
        if (vi < rs.nvec) {
          float f[kVec];
          E::unpack(buf[j], f);
#pragma unroll
          for (int i = 0; i < kVec; ++i) ls += __builtin_amdgcn_exp2f(fmaf(f[i], kLog2e, nm2));
        }
      }
      if (tid < rs.head) ls += __builtin_amdgcn_exp2f(fmaf(E::load(z + tid), kLog2e, nm2));
      if (tid < V - rs.tail0) ls += __builtin_amdgcn_exp2f(fmaf(E::load(z + rs.tail0 + tid), kLog2e, nm2));
    }
    m = lm;
    s = ls;
  } else {
    if (sc.n > 0) count_partial<kThreads>(sc, targets, V, ign, t_first, cnt);
    stream_row<kThreads>(zv, rs.nvec, [&](int64_t, const uint4& v) {
      float f[kVec];
      E::unpack(v, f);
      online_push_vec<kVec>(m, s, f);
    });
    if (tid < rs.head) online_push(m, s, E::load(z + tid));
    if (tid < V - rs.tail0) online_push(m, s, E::load(z + rs.tail0 + tid));
  }

  // The reduction's barriers also publish the per-wave counts.
  float lse;
  if constexpr (kRes > 0) {
    lse = block_lse2<kThreads>(m, s, red0, red1);
  } else {
    float M, S;
    block_lse_parts<kThreads>(m, s, red0, red1, M, S);
    lse = M + __builtin_amdgcn_logf(S) * kLn2;
  }
  if (sc.n > 0) self_scale = count_finish<kThreads>(sc, cnt);
  if constexpr (kRes > 0) zt = E::load(&zt_bits);
  // Loss and per-row factor belong to the original row (packed chunks).
  const int64_t orow = pk.map != nullptr ? static_cast<int64_t>(pk.map[row]) : row;
  if (tid == 0) loss_rows[orow] = valid ? (lse - zt) : 0.0f;
  if (G != nullptr) row_ce_grad<T, kThreads, kRes>(Z, ldz, G, ldg, V, pad_cols, row, y, valid,
                                                  lse, zt, rs, buf, row_scale, orow, grad_shift,
                                                  sc.n > 0 ? self_scale : hdr->scale, sc.nt_grad);
}

// The gradient part of k_row_ce: grad row = c (softmax - onehot), from the
// registers (kRes > 0) or a second streaming pass; pad columns set to zero.
template <typename T, int kThreads, int kRes>
__device__ __forceinline__ void row_ce_grad(const T* Z, int64_t ldz, T* G, int64_t ldg, int64_t V,
                                            int64_t pad_cols, int64_t row, int32_t y, bool valid,
                                            float lse, float zt, const RowSplit& rs, const uint4* buf,
                                            const float* __restrict__ row_scale, int64_t orow,
                                            int grad_shift, float red_scale, int nt) {
  using E = Elem<T>;
  constexpr int kVec = E::kVec;
  const int tid = threadIdx.x;
  const T* z = Z + row * ldz;
  const uint4* zv = reinterpret_cast<const uint4*>(z + rs.head);

  // The gradient factor: the reduction's, or a per-row one (sequence-level
  // losses such as DPO weight each token row separately); with grad_shift
  // the reduction's scale is left to the consumer.
  const float c = !valid ? 0.0f
                  : grad_shift > 0 ? __builtin_ldexpf(row_scale != nullptr ? row_scale[orow] : 1.0f, grad_shift)
                  : (row_scale != nullptr ? row_scale[orow] : red_scale);
  T* g = G + row * ldg;
  uint4* gv = reinterpret_cast<uint4*>(g + rs.head);
  auto grad_of = [&](float x, int64_t v) -> float {
    if (!valid) return 0.0f;
    const float p = __builtin_amdgcn_exp2f((x - lse) * kLog2e);
    return c * (v == y ? p - 1.0f : p);
  };
  // The target's position relative to vector vi's first column, and its
  // gradient (valid rows only, where 0 <= y < V).
  const int rel0 = valid ? y - static_cast<int>(rs.head) : 0;
  const float gt = c * (__builtin_amdgcn_exp2f((zt - lse) * kLog2e) - 1.0f);
  if (!valid) {
    // The whole row (uniform branch): zeros. A plain strided loop, so that
    // no per-vector index of the register-resident loop below is kept live
    // for this rare case.
    const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
    for (int64_t vi = tid; vi < rs.nvec; vi += kThreads) store_grad_vec(gv + vi, zero, nt);
  } else if constexpr (kRes > 0) {
#pragma unroll
    for (int j = 0; j < kRes; ++j) {
      const int64_t vi = static_cast<int64_t>(j) * kThreads + tid;
      if (vi < rs.nvec)
        store_grad_vec(gv + vi, ce_grad_vec<T>(buf[j], rel0 - static_cast<int>(vi) * kVec, c, lse, gt), nt);
    }
  } else {
    stream_row<kThreads, true>(zv, rs.nvec, [&](int64_t vi, const uint4& v) {
      store_grad_vec(gv + vi, ce_grad_vec<T>(v, static_cast<int>(rel0 - vi * kVec), c, lse, gt), nt);
    });
  }
  if (tid < rs.head) E::store(g + tid, grad_of(E::load(z + tid), tid));
  if (tid < V - rs.tail0) {
    const int64_t v = rs.tail0 + tid;
    E::store(g + v, grad_of(E::load(z + v), v));
  }
  if (tid < pad_cols) E::store(g + V + tid, 0.0f);
}

// Persistent variant for long register-resident rows (1024 lanes, kRes
// vectors per lane): one workgroup per CU walks rows blockIdx.x, +gridDim.x,
// ... While a row is reduced and its gradient written, the first kSlices x
// 16 KiB of the workgroup's next row stream into LDS with direct loads, so
// HBM stays busy through the row's compute phase. Each lane reads back only
// the bytes its own direct loads wrote, so the hand-off needs no barrier:
// the compiler's per-wave wait for those loads is enough.
namespace pf {
constexpr int kThreads = 1024;
constexpr int kMaxSlices = 9;  // 144 KiB of LDS
__shared__ __align__(16) uint4 g_next[kMaxSlices * kThreads];
typedef __attribute__((address_space(3))) void lds_void;

}  // namespace pf

template <typename T, int kRes>
__global__ __launch_bounds__(pf::kThreads) void k_row_ce_pf(const T* Z, int64_t ldz, T* G,
                                                            int64_t ldg, int64_t rows, int64_t V,
                                                            int64_t pad_cols,
                                                            const int32_t* __restrict__ targets,
                                                            int32_t ign,
                                                            const WsHeader* __restrict__ hdr,
                                                            float* __restrict__ loss_rows,
                                                            const float* __restrict__ row_scale,
                                                            int grad_shift, RowPack pk) {
  using E = Elem<T>;
  constexpr int kVec = E::kVec;
  constexpr int kThreads = pf::kThreads;
  // Packed chunks: only the live rows exist.
  if (pk.live != nullptr) {
    const int64_t live = static_cast<int64_t>(*pk.live) - pk.base;
    if (live < rows) rows = live;
  }
  constexpr int kSlices = kRes < pf::kMaxSlices ? kRes : pf::kMaxSlices;
  __shared__ float red0[kThreads / 64], red1[kThreads / 64];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // Direct loads of slices 0..kSlices-1 of `row` (vector j*kThreads + tid to
  // LDS slot j*kThreads + tid); vectors past the row read as zero.
  auto prefetch = [&](int64_t row) {
    const T* z = Z + row * ldz;
    const RowSplit rs = split_row(z, V);
    const __amdgpu_buffer_rsrc_t r = row_rsrc(z + rs.head, rs.nvec * 16);
#pragma unroll
    for (int j = 0; j < kSlices; ++j)  // slice offset in the scalar offset register
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (pf::lds_void*)(&pf::g_next[j * kThreads + wave * 64]), 16, tid * 16,
          j * kThreads * 16, 0, 0);
  };

  int64_t row = blockIdx.x;
  if (row >= rows) return;
  prefetch(row);
  for (; row < rows; row += gridDim.x) {
    const T* z = Z + row * ldz;
    const int32_t y = targets[row];
    const bool valid = (y != ign) && y >= 0 && static_cast<int64_t>(y) < V;
    const RowSplit rs = split_row(z, V);
    // Here V <= 16 * 1024 vectors: 32-bit element and vector indices.
    const int nvec = static_cast<int>(rs.nvec), head = static_cast<int>(rs.head);
    const int tail0 = static_cast<int>(rs.tail0), Vi = static_cast<int>(V);
    float zt = 0.0f;
    if (valid) zt = E::load(z + y);  // every lane, before any lane overwrites the row

    uint4 buf[kRes];
    {
      const __amdgpu_buffer_rsrc_t r = row_rsrc(z + head, rs.nvec * 16);
#pragma unroll
      for (int j = kSlices; j < kRes; ++j)  // range-checked: zeros past the row
        buf[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                               r, tid * 16, j * kThreads * 16, 0));
    }
#pragma unroll
    for (int j = 0; j < kSlices; ++j) buf[j] = pf::g_next[j * kThreads + tid];
    // The LDS slots are reloaded next: the reads above must have completed.
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
    if (row + gridDim.x < rows) prefetch(row + gridDim.x);

    float lm = -INFINITY;
#pragma unroll
    for (int j = 0; j < kRes; ++j) {
      if (j * kThreads + tid < nvec) {
        float f[kVec];
        E::unpack(buf[j], f);
#pragma unroll
        for (int i = 0; i < kVec; ++i) lm = fmaxf(lm, f[i]);
      }
    }
    if (tid < head) lm = fmaxf(lm, E::load(z + tid));
    if (tid < Vi - tail0) lm = fmaxf(lm, E::load(z + tail0 + tid));
    // Base-2 sum against the lane maximum (block_lse2).
    float ls = 0.0f;
    if (lm != -INFINITY) {
      const float nm2 = -lane_m2(lm);
#pragma unroll
      for (int j = 0; j < kRes; ++j) {
        if (j * kThreads + tid < nvec) {
          float f[kVec];
          E::unpack(buf[j], f);
#pragma unroll
          for (int i = 0; i < kVec; ++i) ls += __builtin_amdgcn_exp2f(fmaf(f[i], kLog2e, nm2));
        }
      }
      if (tid < head) ls += __builtin_amdgcn_exp2f(fmaf(E::load(z + tid), kLog2e, nm2));
      if (tid < Vi - tail0) ls += __builtin_amdgcn_exp2f(fmaf(E::load(z + tail0 + tid), kLog2e, nm2));
    }
    const float lse = block_lse2<kThreads>(lm, ls, red0, red1);
    const int64_t orow = pk.map != nullptr ? static_cast<int64_t>(pk.map[row]) : row;
    if (tid == 0) loss_rows[orow] = valid ? (lse - zt) : 0.0f;

    if (G != nullptr) {
      const float c = !valid ? 0.0f
                      : grad_shift > 0 ? __builtin_ldexpf(row_scale != nullptr ? row_scale[orow] : 1.0f, grad_shift)
                      : (row_scale != nullptr ? row_scale[orow] : hdr->scale);
      const int yt = valid ? y : -1;
      T* g = G + row * ldg;
      uint4* gv = reinterpret_cast<uint4*>(g + head);
      auto grad_of = [&](float x, int v) -> float {
        if (!valid) return 0.0f;
        const float p = __builtin_amdgcn_exp2f((x - lse) * kLog2e);
        return c * (v == yt ? p - 1.0f : p);
      };
      if (!valid) {
        // The whole row (uniform branch): zeros.
        for (int vi = tid; vi < nvec; vi += kThreads) gv[vi] = make_uint4(0u, 0u, 0u, 0u);
      } else {
        const int rel0 = y - head;
        const float gt = c * (__builtin_amdgcn_exp2f((zt - lse) * kLog2e) - 1.0f);
#pragma unroll
        for (int j = 0; j < kRes; ++j) {
          const int vi = j * kThreads + tid;
          if (vi < nvec) gv[vi] = ce_grad_vec<T>(buf[j], rel0 - vi * kVec, c, lse, gt);
        }
      }
      if (tid < head) E::store(g + tid, grad_of(E::load(z + tid), tid));
      if (tid < Vi - tail0) E::store(g + tail0 + tid, grad_of(E::load(z + tail0 + tid), tail0 + tid));
      if (tid < pad_cols) E::store(g + V + tid, 0.0f);
    }
    __syncthreads();  // red0 / red1 are rewritten by the next row
  }
  // Direct loads past the last row would still be in flight here; none are
  // issued for rows >= rows.
}

static int cu_count() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      cus = n;
    else
      return 256;
  }
  return cus;
}

// Rows of 8193..16384 16-byte vectors (1024-lane workgroups), at least two
// per CU: the persistent prefetching kernel.
static bool takes_persistent(int64_t nvec, int64_t rows) {
  return nvec > 8 * pf::kThreads && nvec <= 16 * pf::kThreads && rows >= 2 * cu_count();
}

template <typename T, int kThreads>
static hipError_t row_ce_dispatch(const void* Z, int64_t ldz, void* G, int64_t ldg, int64_t rows,
                                  int64_t V, int64_t pad_cols, const int32_t* targets, int32_t ign,
                                  const WsHeader* hdr, float* loss_rows, const float* row_scale,
                                  int grad_shift, SelfCount sc, RowPack pk, hipStream_t s) {
  constexpr int kVec = Elem<T>::kVec;
  const int64_t nvec_max = (V + kVec - 1) / kVec;
  const T* z = static_cast<const T*>(Z);
  T* g = static_cast<T*>(G);
  const dim3 grid(static_cast<unsigned>(rows)), block(kThreads);
#define LCE_ROW_CE(R)                                                                           \
  hipLaunchKernelGGL((k_row_ce<T, kThreads, R>), grid, block, 0, s, z, ldz, g, ldg, V, pad_cols, \
                     targets, ign, hdr, loss_rows, row_scale, grad_shift, sc, pk)
  // Long rows, more rows than CUs: the persistent prefetching variant.
  if constexpr (kThreads == pf::kThreads) {
    if (sc.n == 0 && takes_persistent(nvec_max, rows)) {
      hipLaunchKernelGGL((k_row_ce_pf<T, 16>), dim3(static_cast<unsigned>(cu_count())), block, 0, s,
                         z, ldz, g, ldg, rows, V, pad_cols, targets, ign, hdr, loss_rows, row_scale,
                         grad_shift, pk);
      return hipGetLastError();
    }
  }
  if (nvec_max <= 1 * kThreads) LCE_ROW_CE(1);
  else if (nvec_max <= 2 * kThreads) LCE_ROW_CE(2);
  else if (nvec_max <= 4 * kThreads) LCE_ROW_CE(4);
  else if (nvec_max <= 8 * kThreads) LCE_ROW_CE(8);
  else if (nvec_max <= 16 * kThreads) LCE_ROW_CE(16);
  else LCE_ROW_CE(0);
#undef LCE_ROW_CE
  return hipGetLastError();
}

template <typename T>
static hipError_t row_ce_by_width(const void* Z, int64_t ldz, void* G, int64_t ldg, int64_t rows,
                                  int64_t V, int64_t pad_cols, const int32_t* targets, int32_t ign,
                                  const WsHeader* hdr, float* loss_rows, const float* row_scale,
                                  int grad_shift, SelfCount sc, RowPack pk, hipStream_t s) {
  if (V >= 16384)
    return row_ce_dispatch<T, 1024>(Z, ldz, G, ldg, rows, V, pad_cols, targets, ign, hdr, loss_rows,
                                    row_scale, grad_shift, sc, pk, s);
  return row_ce_dispatch<T, 256>(Z, ldz, G, ldg, rows, V, pad_cols, targets, ign, hdr, loss_rows,
                                 row_scale, grad_shift, sc, pk, s);
}

static hipError_t row_ce_typed(int dtype, const void* Z, int64_t ldz, void* G, int64_t ldg,
                               int64_t rows, int64_t V, int64_t pad_cols, const int32_t* targets,
                               int32_t ign, const WsHeader* hdr, float* loss_rows,
                               const float* row_scale, int grad_shift, SelfCount sc,
                               RowPack pk, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (dtype == 1)
    return row_ce_by_width<uint16_t>(Z, ldz, G, ldg, rows, V, pad_cols, targets, ign, hdr,
                                     loss_rows, row_scale, grad_shift, sc, pk, s);
  if (dtype == 2)
    return row_ce_by_width<Half>(Z, ldz, G, ldg, rows, V, pad_cols, targets, ign, hdr, loss_rows,
                                 row_scale, grad_shift, sc, pk, s);
  return row_ce_by_width<float>(Z, ldz, G, ldg, rows, V, pad_cols, targets, ign, hdr, loss_rows,
                                row_scale, grad_shift, sc, pk, s);
}

hipError_t launch_row_ce(int dtype, const void* Z, int64_t ldz, void* G, int64_t ldg, int64_t rows,
                         int64_t V, int64_t pad_cols, const int32_t* targets, int32_t ign,
                         const WsHeader* hdr, float* loss_rows, const float* row_scale,
                         int grad_shift, hipStream_t s, RowPack pk) {
  return row_ce_typed(dtype, Z, ldz, G, ldg, rows, V, pad_cols, targets, ign, hdr, loss_rows,
                      row_scale, grad_shift, SelfCount{0, 0, nullptr, 0}, pk, s);
}

// Standalone calls (one launch, the targets counted here): two register-
// resident rows per workgroup. Both rows' loads go out before either is
// used, so the first row's reductions and gradient stores run while the
// second row is still arriving. The targets the count needs are loaded
// before the rows (loads complete in order: a target load issued after the
// rows would wait for both).
template <typename T, int kThreads, int kRes>
__global__ __launch_bounds__(kThreads) void k_row_ce_pair(const T* Z, T* G, int64_t rows, int64_t V,
                                                          const int32_t* __restrict__ targets,
                                                          int32_t ign, float* __restrict__ loss_rows,
                                                          SelfCount sc) {
  using E = Elem<T>;
  constexpr int kVec = E::kVec;
  constexpr int kCnt = 4;  // targets per lane for the count: 4 x 512 = the self-count limit
  __shared__ float red0[kThreads / 64], red1[kThreads / 64];
  __shared__ float cnt[2][kThreads / 64];
  const int tid = threadIdx.x;
  int32_t tc[kCnt];
#pragma unroll
  for (int k = 0; k < kCnt; ++k) tc[k] = tid + k * kThreads < sc.n ? targets[tid + k * kThreads] : ign;
  const int64_t r0 = 2 * static_cast<int64_t>(blockIdx.x);
  const bool two = r0 + 1 < rows;
  const int32_t y0 = targets[r0], y1 = two ? targets[r0 + 1] : ign;
  const bool v0 = y0 != ign && y0 >= 0 && static_cast<int64_t>(y0) < V;
  const bool v1 = two && y1 != ign && y1 >= 0 && static_cast<int64_t>(y1) < V;
  const T* z0 = Z + r0 * V;
  const T* z1 = z0 + V;
  const RowSplit rs0 = split_row(z0, V), rs1 = split_row(z1, V);
  uint4 b0[kRes], b1[kRes];
  T t0{}, t1{};
  {
    const __amdgpu_buffer_rsrc_t a = row_rsrc(z0 + rs0.head, rs0.nvec * 16);
#pragma unroll
    for (int j = 0; j < kRes; ++j)
      b0[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(a, (j * kThreads + tid) * 16, 0, 0));
    t0 = load_elem_bits<T>(row_rsrc(z0, V * static_cast<int64_t>(sizeof(T))),
                           v0 ? static_cast<int>(y0 * sizeof(T)) : 0x7FFFFFF0);
    const __amdgpu_buffer_rsrc_t b = row_rsrc(z1 + rs1.head, two ? rs1.nvec * 16 : 0);
#pragma unroll
    for (int j = 0; j < kRes; ++j)
      b1[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(b, (j * kThreads + tid) * 16, 0, 0));
    t1 = load_elem_bits<T>(row_rsrc(z1, two ? V * static_cast<int64_t>(sizeof(T)) : 0),
                           v1 ? static_cast<int>(y1 * sizeof(T)) : 0x7FFFFFF0);
  }
  {
    int valid = 0, bad = 0;
#pragma unroll
    for (int k = 0; k < kCnt; ++k) {
      const int32_t y = tc[k];
      if (y != ign) {
        if (y >= 0 && static_cast<int64_t>(y) < V) ++valid; else ++bad;
      }
    }
    const float fv = wave_sum(static_cast<float>(valid)), fb = wave_sum(static_cast<float>(bad));
    if ((tid & 63) == 0) {
      cnt[0][tid >> 6] = fv;
      cnt[1][tid >> 6] = fb;
    }
  }
  float scale = 0.0f;
  auto row = [&](const T* z, int64_t r, int32_t y, bool valid, const RowSplit& rs,
                 const uint4 (&buf)[kRes], T tb, bool first) {
    float lm = -INFINITY;
#pragma unroll
    for (int j = 0; j < kRes; ++j) {
      if (static_cast<int64_t>(j) * kThreads + tid < rs.nvec) {
        float f[kVec];
        E::unpack(buf[j], f);
#pragma unroll
        for (int i = 0; i < kVec; ++i) lm = fmaxf(lm, f[i]);
      }
    }
    if (tid < rs.head) lm = fmaxf(lm, E::load(z + tid));
    if (tid < V - rs.tail0) lm = fmaxf(lm, E::load(z + rs.tail0 + tid));
    float ls = 0.0f;
    if (lm != -INFINITY) {
      const float nm2 = -lane_m2(lm);
#pragma unroll
      for (int j = 0; j < kRes; ++j) {
        if (static_cast<int64_t>(j) * kThreads + tid < rs.nvec) {
          float f[kVec];
          E::unpack(buf[j], f);
#pragma unroll
          for (int i = 0; i < kVec; ++i) ls += __builtin_amdgcn_exp2f(fmaf(f[i], kLog2e, nm2));
        }
      }
      if (tid < rs.head) ls += __builtin_amdgcn_exp2f(fmaf(E::load(z + tid), kLog2e, nm2));
      if (tid < V - rs.tail0) ls += __builtin_amdgcn_exp2f(fmaf(E::load(z + rs.tail0 + tid), kLog2e, nm2));
    }
    // The first row's barriers also publish the per-wave counts.
    const float lse = block_lse2<kThreads>(lm, ls, red0, red1);
    if (first) scale = count_finish<kThreads>(sc, cnt);
    const float zt = E::load(&tb);
    if (tid == 0) loss_rows[r] = valid ? (lse - zt) : 0.0f;
    if (G != nullptr)
      row_ce_grad<T, kThreads, kRes>(Z, V, G, V, V, 0, r, y, valid, lse, zt, rs, buf, nullptr, r, 0,
                                     scale, sc.nt_grad);
  };
  row(z0, r0, y0, v0, rs0, b0, t0, true);
  if (two) {
    __syncthreads();  // red0 / red1 are reused
    row(z1, r0 + 1, y1, v1, rs1, b1, t1, false);
  }
}

// Standalone calls of rows of up to 8192 16-byte vectors: 512-lane
// workgroups. Rows of up to 4096 vectors (the [1024, 32768] bf16 shard: 8
// per lane) go two to a workgroup (k_row_ce_pair: 114 VGPRs, two workgroups
// and so every row of the shard resident per CU; the first row's reductions
// and stores overlap the second row's loads): 26.5-26.9 against 28.5-29.0 us
// for the kernel alone with one row per workgroup (70 VGPRs, three
// workgroups per CU). Earlier, one row per workgroup: 256-lane workgroups of
// 16 vectors (four per CU) measured slower than 512 lanes (33-34 against
// 32-33 us per call), and so did 512 lanes held to 64 VGPRs for four
// workgroups per CU (30.6-31.2 against 27.7-28.3 us for the kernel).
template <typename T>
static bool row_ce_512(const void* Z, void* G, int64_t rows, int64_t V, const int32_t* targets,
                       int32_t ign, const WsHeader* hdr, float* loss_rows, SelfCount sc,
                       hipStream_t s) {
  constexpr int kVec = Elem<T>::kVec;
  const int64_t nvec = (V + kVec - 1) / kVec;
  const T* z = static_cast<const T*>(Z);
  T* g = static_cast<T*>(G);
  const dim3 block(512);
  if (sc.n > 4 * 512) return false;  // the pair kernel holds 4 targets per lane for the count
  if (nvec <= 8 * 512) {
    const dim3 grid(static_cast<unsigned>((rows + 1) / 2));
    if (nvec <= 4 * 512)
      hipLaunchKernelGGL((k_row_ce_pair<T, 512, 4>), grid, block, 0, s, z, g, rows, V, targets, ign,
                         loss_rows, sc);
    else
      hipLaunchKernelGGL((k_row_ce_pair<T, 512, 8>), grid, block, 0, s, z, g, rows, V, targets, ign,
                         loss_rows, sc);
    return true;
  }
  if (nvec > 16 * 512) return false;
  const RowPack pk{nullptr, nullptr, 0};
  hipLaunchKernelGGL((k_row_ce<T, 512, 16>), dim3(static_cast<unsigned>(rows)), block, 0, s, z, V, g,
                     V, V, int64_t(0), targets, ign, hdr, loss_rows, static_cast<const float*>(nullptr),
                     0, sc, pk);
  return true;
}

hipError_t launch_row_ce_counted(int dtype, const void* Z, void* G, int64_t rows, int64_t V,
                                 const int32_t* targets, int32_t ign, int reduction, WsHeader* hdr,
                                 float* loss_rows, hipStream_t s) {
  // Rows that the persistent prefetching kernel takes (it does not count)
  // keep the separate count launch.
  const int vec = dtype == 0 ? 4 : 8;  // elements per 16-byte vector
  if (V >= 16384 && takes_persistent((V + vec - 1) / vec, rows)) {
    const hipError_t e = launch_count_targets(targets, rows, V, ign, reduction, hdr, s);
    if (e != hipSuccess) return e;
    return launch_row_ce(dtype, Z, V, G, V, rows, V, 0, targets, ign, hdr, loss_rows, nullptr, 0, s);
  }
  const SelfCount sc{rows, reduction, hdr, 1};
  hipError_t e = hipSuccess;
  bool done = false;
  if (V >= 16384) {
    if (dtype == 1) done = row_ce_512<uint16_t>(Z, G, rows, V, targets, ign, hdr, loss_rows, sc, s);
    else if (dtype == 2) done = row_ce_512<Half>(Z, G, rows, V, targets, ign, hdr, loss_rows, sc, s);
    else done = row_ce_512<float>(Z, G, rows, V, targets, ign, hdr, loss_rows, sc, s);
    if (done) e = hipGetLastError();
  }
  if (!done)
    e = row_ce_typed(dtype, Z, V, G, V, rows, V, 0, targets, ign, hdr, loss_rows, nullptr, 0, sc,
                     RowPack{nullptr, nullptr, 0}, s);
  return e;
}

// ------------------------------------------------------------ shard stats

// kRes > 0: the row's vectors are loaded at once into registers (kRes per
// lane), as in k_row_ce; kRes == 0: one streaming online pass.
template <typename T, int kThreads, int kRes>
__global__ __launch_bounds__(kThreads) void k_shard_stats(const T* __restrict__ Z, int64_t ldz,
                                                          int64_t Vl, int64_t v0, int64_t Vg,
                                                          const int32_t* __restrict__ targets,
                                                          int32_t ign, float* __restrict__ rmax,
                                                          float* __restrict__ rsum,
                                                          float* __restrict__ rtgt, SelfCount sc) {
  using E = Elem<T>;
  constexpr int kVec = E::kVec;
  __shared__ float red0[kThreads / 64], red1[kThreads / 64];
  __shared__ float cnt[2][kThreads / 64];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const T* z = Z + row * ldz;
  const int32_t y = targets[row];
  const int64_t local = static_cast<int64_t>(y) - v0;
  const bool here = (y != ign) && y >= 0 && static_cast<int64_t>(y) < Vg && local >= 0 && local < Vl;
  const RowSplit rs = split_row(z, Vl);
  const uint4* zv = reinterpret_cast<const uint4*>(z + rs.head);
  const int32_t t_first = (sc.n > 0 && tid < sc.n) ? targets[tid] : ign;
  float m = -INFINITY, s = 0.0f, zt = 0.0f;
  if constexpr (kRes > 0) {
    // As in k_row_ce: branch-free loads, then the target element; rows here
    // hold at most 16 x kThreads vectors, so byte offsets fit in 32 bits.
    const __amdgpu_buffer_rsrc_t rv = row_rsrc(zv, rs.nvec * 16);
    uint4 buf[kRes];
#pragma unroll
    for (int j = 0; j < kRes; ++j)
      buf[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                              rv, (j * kThreads + tid) * 16, 0, 0));
    const T zt_bits = load_elem_bits<T>(row_rsrc(z, Vl * static_cast<int64_t>(sizeof(T))),
                                        here ? static_cast<int>(local * sizeof(T)) : 0x7FFFFFF0);
    if (sc.n > 0) count_partial<kThreads>(sc, targets, Vg, ign, t_first, cnt);
    float lm = -INFINITY;
#pragma unroll
    for (int j = 0; j < kRes; ++j) {
      if (j * kThreads + tid < rs.nvec) {
        float f[kVec];
        E::unpack(buf[j], f);
#pragma unroll
        for (int i = 0; i < kVec; ++i) lm = fmaxf(lm, f[i]);
      }
    }
    if (tid < rs.head) lm = fmaxf(lm, E::load(z + tid));
    if (tid < Vl - rs.tail0) lm = fmaxf(lm, E::load(z + rs.tail0 + tid));
    float ls = 0.0f;
    if (lm != -INFINITY) {
#pragma unroll
      for (int j = 0; j < kRes; ++j) {
        if (j * kThreads + tid < rs.nvec) {
          float f[kVec];
          E::unpack(buf[j], f);
#pragma unroll
          for (int i = 0; i < kVec; ++i) ls += __builtin_amdgcn_exp2f((f[i] - lm) * kLog2e);
        }
      }
      if (tid < rs.head) ls += __builtin_amdgcn_exp2f((E::load(z + tid) - lm) * kLog2e);
      if (tid < Vl - rs.tail0) ls += __builtin_amdgcn_exp2f((E::load(z + rs.tail0 + tid) - lm) * kLog2e);
    }
    m = lm;
    s = ls;
    zt = E::load(&zt_bits);
  } else {
    if (sc.n > 0) count_partial<kThreads>(sc, targets, Vg, ign, t_first, cnt);
    stream_row<kThreads>(zv, rs.nvec, [&](int64_t, const uint4& v) {
      float f[kVec];
      E::unpack(v, f);
      online_push_vec<kVec>(m, s, f);
    });
    if (tid < rs.head) online_push(m, s, E::load(z + tid));
    if (tid < Vl - rs.tail0) online_push(m, s, E::load(z + rs.tail0 + tid));
    if (tid == 0 && here) zt = E::load(z + local);
  }
  // The reduction's barriers also publish the per-wave counts.
  float M, S;
  block_lse_parts<kThreads>(m, s, red0, red1, M, S);
  if (sc.n > 0) count_finish<kThreads>(sc, cnt);
  if (tid == 0) {
    rmax[row] = M;
    rsum[row] = S;
    rtgt[row] = here ? zt : 0.0f;
  }
}

template <typename T>
static hipError_t shard_stats_typed(const void* Z, int64_t ldz, int64_t rows, int64_t Vl,
                                    int64_t v0, int64_t Vg, const int32_t* targets, int32_t ign,
                                    float* rmax, float* rsum, float* rtgt, SelfCount sc,
                                    hipStream_t s) {
  constexpr int kThreads = 1024;
  const int64_t nvec_max = (Vl + Elem<T>::kVec - 1) / Elem<T>::kVec;
  const T* z = static_cast<const T*>(Z);
  const dim3 grid(static_cast<unsigned>(rows)), block(kThreads);
#define LCE_SHARD(R)                                                                            \
  hipLaunchKernelGGL((k_shard_stats<T, kThreads, R>), grid, block, 0, s, z, ldz, Vl, v0, Vg,     \
                     targets, ign, rmax, rsum, rtgt, sc)
  if (nvec_max <= 1 * kThreads) LCE_SHARD(1);
  else if (nvec_max <= 2 * kThreads) LCE_SHARD(2);
  else if (nvec_max <= 4 * kThreads) LCE_SHARD(4);
  else if (nvec_max <= 8 * kThreads) LCE_SHARD(8);
  else if (nvec_max <= 16 * kThreads) LCE_SHARD(16);
  else LCE_SHARD(0);
#undef LCE_SHARD
  return hipGetLastError();
}

static hipError_t shard_stats_any(int dtype, const void* Z, int64_t ldz, int64_t rows,
                                  int64_t V_local, int64_t vocab_start, int64_t V_global,
                                  const int32_t* targets, int32_t ign, float* row_max,
                                  float* row_sumexp, float* row_target, SelfCount sc,
                                  hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (dtype == 1)
    return shard_stats_typed<uint16_t>(Z, ldz, rows, V_local, vocab_start, V_global, targets, ign,
                                       row_max, row_sumexp, row_target, sc, s);
  if (dtype == 2)
    return shard_stats_typed<Half>(Z, ldz, rows, V_local, vocab_start, V_global, targets, ign,
                                   row_max, row_sumexp, row_target, sc, s);
  return shard_stats_typed<float>(Z, ldz, rows, V_local, vocab_start, V_global, targets, ign,
                                  row_max, row_sumexp, row_target, sc, s);
}

hipError_t launch_shard_stats(int dtype, const void* Z, int64_t ldz, int64_t rows, int64_t V_local,
                              int64_t vocab_start, int64_t V_global, const int32_t* targets,
                              int32_t ign, float* row_max, float* row_sumexp, float* row_target,
                              hipStream_t s) {
  return shard_stats_any(dtype, Z, ldz, rows, V_local, vocab_start, V_global, targets, ign,
                         row_max, row_sumexp, row_target, SelfCount{0, 0, nullptr, 0}, s);
}

hipError_t launch_shard_stats_counted(int dtype, const void* Z, int64_t rows, int64_t V_local,
                                      int64_t vocab_start, int64_t V_global,
                                      const int32_t* targets, int32_t ign, float* row_max,
                                      float* row_sumexp, float* row_target, WsHeader* hdr,
                                      hipStream_t s) {
  return shard_stats_any(dtype, Z, V_local, rows, V_local, vocab_start, V_global, targets, ign,
                         row_max, row_sumexp, row_target, SelfCount{rows, 1, hdr, 0}, s);
}

// ------------------------------------------------- vocabulary-shard backward

// In place over one shard's logits [rows, V_local] (global ids v0 + j), given
// the global lse of each row: dZ = c * (exp(z - lse) - [v0 + j == y]) with
// c = the reduction scale (2^grad_shift instead when grad_shift > 0) for rows
// valid w.r.t. V_global, 0 otherwise. One
// read and one write per element; pad columns [V_local, V_local + pad) are
// zeroed for the GEMMs that read the chunk.
template <typename T, int kThreads>
__global__ __launch_bounds__(kThreads) void k_shard_grad(T* Z, int64_t ldz, int64_t Vl,
                                                         int64_t pad_cols, int64_t v0, int64_t Vg,
                                                         const int32_t* __restrict__ targets,
                                                         int32_t ign, const float* __restrict__ lse,
                                                         const WsHeader* __restrict__ hdr,
                                                         int grad_shift, RowPack pk) {
  using E = Elem<T>;
  constexpr int kVec = E::kVec;
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  // Packed chunks: rows past the live count do not exist (whole workgroup).
  if (pk.live != nullptr && row >= static_cast<int64_t>(*pk.live) - pk.base) return;
  T* z = Z + row * ldz;
  const int32_t y = targets[row];
  const bool valid = (y != ign) && y >= 0 && static_cast<int64_t>(y) < Vg;
  const float c = !valid ? 0.0f : grad_shift > 0 ? __builtin_ldexpf(1.0f, grad_shift) : hdr->scale;
  const float L = lse[pk.map != nullptr ? static_cast<int64_t>(pk.map[row]) : row];
  const int64_t jt = valid ? static_cast<int64_t>(y) - v0 : -1;  // may fall outside the shard
  auto grad_of = [&](float x, int64_t j) -> float {
    if (!valid) return 0.0f;
    const float p = __builtin_amdgcn_exp2f((x - L) * kLog2e);
    return c * (j == jt ? p - 1.0f : p);
  };
  const RowSplit rs = split_row(z, Vl);
  uint4* zv = reinterpret_cast<uint4*>(z + rs.head);
  if (!valid) {
    // The whole row (uniform branch): zeros.
    for (int64_t vi = tid; vi < rs.nvec; vi += kThreads) zv[vi] = make_uint4(0u, 0u, 0u, 0u);
  } else {
    // The target's gradient, from its logit when the target is in this shard:
    // every lane reads it, and the barrier keeps those reads ahead of the
    // lanes' writes (a workgroup's memory operations issue in order on its
    // CU). rel0 falls outside every vector when the target is not here
    // (|jt| < 2^30).
    const bool here = jt >= 0 && jt < Vl;
    const float zt = here ? E::load(z + jt) : 0.0f;
    __syncthreads();
    const float gt = c * (__builtin_amdgcn_exp2f((zt - L) * kLog2e) - 1.0f);
    const int64_t rel0 = jt - rs.head;
    stream_row<kThreads>(zv, rs.nvec, [&](int64_t vi, const uint4& v) {
      zv[vi] = ce_grad_vec<T>(v, static_cast<int>(rel0 - vi * kVec), c, L, gt);
    });
  }
  if (tid < rs.head) E::store(z + tid, grad_of(E::load(z + tid), tid));
  if (tid < Vl - rs.tail0) {
    const int64_t j = rs.tail0 + tid;
    E::store(z + j, grad_of(E::load(z + j), j));
  }
  if (tid < pad_cols) E::store(z + Vl + tid, 0.0f);
}

hipError_t launch_shard_grad(int dtype, void* Z, int64_t ldz, int64_t rows, int64_t V_local,
                             int64_t pad_cols, int64_t vocab_start, int64_t V_global,
                             const int32_t* targets, int32_t ign, const float* lse,
                             const WsHeader* hdr, int grad_shift, hipStream_t s, RowPack pk) {
  if (rows <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(rows));
  if (dtype == 1)
    hipLaunchKernelGGL((k_shard_grad<uint16_t, 256>), grid, dim3(256), 0, s, static_cast<uint16_t*>(Z),
                       ldz, V_local, pad_cols, vocab_start, V_global, targets, ign, lse, hdr,
                       grad_shift, pk);
  else if (dtype == 2)
    hipLaunchKernelGGL((k_shard_grad<Half, 256>), grid, dim3(256), 0, s, static_cast<Half*>(Z), ldz,
                       V_local, pad_cols, vocab_start, V_global, targets, ign, lse, hdr, grad_shift, pk);
  else
    hipLaunchKernelGGL((k_shard_grad<float, 256>), grid, dim3(256), 0, s, static_cast<float*>(Z), ldz,
                       V_local, pad_cols, vocab_start, V_global, targets, ign, lse, hdr, grad_shift, pk);
  return hipGetLastError();
}

// Combine P shards' (max, sumexp, target logit) per row, shards in index
// order, in float64: M = max m_k, lse = M + ln sum_k s_k exp(m_k - M),
// z_y = sum_k t_k; loss row = lse - z_y for valid rows, 0 otherwise.
__global__ __launch_bounds__(256) void k_combine_stats(const float* __restrict__ ms,
                                                       const float* __restrict__ ss,
                                                       const float* __restrict__ ts, int64_t P,
                                                       int64_t N, const int32_t* __restrict__ targets,
                                                       int32_t ign, int64_t Vg,
                                                       float* __restrict__ lse_out,
                                                       float* __restrict__ loss_rows) {
  const int64_t n = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (n >= N) return;
  double M = -INFINITY;
  for (int64_t k = 0; k < P; ++k) M = fmax(M, static_cast<double>(ms[k * N + n]));
  double S = 0.0, t = 0.0;
  for (int64_t k = 0; k < P; ++k) {
    S += static_cast<double>(ss[k * N + n]) * exp(static_cast<double>(ms[k * N + n]) - M);
    t += static_cast<double>(ts[k * N + n]);
  }
  const double lse = M + log(S);
  const int32_t y = targets[n];
  const bool valid = (y != ign) && y >= 0 && static_cast<int64_t>(y) < Vg;
  if (lse_out != nullptr) lse_out[n] = static_cast<float>(lse);
  loss_rows[n] = valid ? static_cast<float>(lse - t) : 0.0f;
}

hipError_t launch_combine_stats(const float* ms, const float* ss, const float* ts, int64_t P,
                                int64_t N, const int32_t* targets, int32_t ign, int64_t V_global,
                                float* lse, float* loss_rows, hipStream_t s) {
  if (N <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_combine_stats, dim3(static_cast<unsigned>((N + 255) / 256)), dim3(256), 0, s,
                     ms, ss, ts, P, N, targets, ign, V_global, lse, loss_rows);
  return hipGetLastError();
}

// ------------------------------------------------------ JSD distillation

// One row of the Jensen-Shannon distillation loss from the student logits S
// and the teacher logits T of the same row (both [V], same type), temperature
// tau: with ls = log softmax(S / tau), lt = log softmax(T / tau) and
// lm = ln((e^ls + e^lt) / 2), loss = 1/2 sum(e^ls (ls - lm)) + 1/2
// sum(e^lt (lt - lm)); the student gradient overwrites S:
// dS = c / tau * e^ls * (g - sum(e^ls g)), g = 1/2 (ls - lm), c the
// reduction scale (0 for masked rows). Three streaming passes: the two
// row statistics, the loss and sum(e^ls g), the gradient.
template <typename T, int kThreads>
__global__ __launch_bounds__(kThreads) void k_row_jsd(T* S, const T* Tt, int64_t ld, int64_t V,
                                                      int64_t pad_cols, float inv_tau,
                                                      const int32_t* __restrict__ targets,
                                                      int32_t ign, const WsHeader* __restrict__ hdr,
                                                      float* __restrict__ loss_rows, int grad_shift,
                                                      RowPack pk) {
  using E = Elem<T>;
  constexpr int kVec = E::kVec;
  __shared__ float red0[kThreads / 64], red1[kThreads / 64];
  const int64_t row = blockIdx.x;
  // Packed chunks: rows past the live count do not exist (whole workgroup).
  if (pk.live != nullptr && row >= static_cast<int64_t>(*pk.live) - pk.base) return;
  const int tid = threadIdx.x;
  T* s = S + row * ld;
  const T* t = Tt + row * ld;
  const int32_t y = targets[row];
  const bool valid = (y != ign) && y >= 0 && static_cast<int64_t>(y) < V;
  // The two buffers share one row stride, so both rows split alike.
  const RowSplit rs = split_row(static_cast<const T*>(s), V);
  const uint4* sv = reinterpret_cast<const uint4*>(s + rs.head);
  const uint4* tv = reinterpret_cast<const uint4*>(t + rs.head);

  // Everything in base 2: u = x k with k = log2(e) / tau for a raw logit x,
  // so 2^u = e^(x / tau).
  const float k2 = lane_m2(inv_tau);

  // Pass 1: per-lane online (max, sum of 2^(u - max)) of both rows; a lane's
  // max is the rounded product of its largest raw logit, the shift its fmas
  // subtract.
  float ms = -INFINITY, ss = 0.0f, mt = -INFINITY, st = 0.0f;
  auto push = [&](float& m, float& sum, const float* x, int n) {
    float vm = x[0];
    for (int i = 1; i < n; ++i) vm = fmaxf(vm, x[i]);
    const float mn = fmaxf(m, lane_m2_by(vm, k2));
    float acc = m == -INFINITY ? 0.0f : sum * __builtin_amdgcn_exp2f(m - mn);
    for (int i = 0; i < n; ++i) acc += __builtin_amdgcn_exp2f(fmaf(x[i], k2, -mn));
    sum = acc;
    m = mn;
  };
  for (int64_t vi = tid; vi < rs.nvec; vi += kThreads) {
    float a[kVec], b[kVec];
    E::unpack(sv[vi], a);
    E::unpack(tv[vi], b);
    push(ms, ss, a, kVec);
    push(mt, st, b, kVec);
  }
  auto scalar_at = [&](int64_t v, float& a, float& b) {
    a = E::load(s + v);
    b = E::load(t + v);
  };
  if (tid < rs.head) { float a, b; scalar_at(tid, a, b); push(ms, ss, &a, 1); push(mt, st, &b, 1); }
  if (tid < V - rs.tail0) {
    float a, b;
    scalar_at(rs.tail0 + tid, a, b);
    push(ms, ss, &a, 1);
    push(mt, st, &b, 1);
  }
  // Row log-sum-exps of u (base 2).
  auto lse2_of = [&](float m, float sum) {
    const float M = block_max<kThreads>(m, red0);
    const float mine = m == -INFINITY ? 0.0f : sum * __builtin_amdgcn_exp2f(m - M);
    return M + __builtin_amdgcn_logf(block_sum<kThreads>(mine, red1));
  };
  const float ls2 = lse2_of(ms, ss);
  __syncthreads();
  const float lt2 = lse2_of(mt, st);

  // Per element, in base 2: P = log2 p, Q = log2 q (the tempered log-softmax
  // of each row over ln 2), LM = log2((p + q) / 2) = max(P, Q) +
  // log2((1 + 2^-|P - Q|) / 2), which cannot underflow; p and q come from
  // 2^max(P, Q) and 2^-|P - Q|: two exponentials and one logarithm per
  // element. Returns dP = P - LM (and dQ, p, q); ln p - ln m = dP ln 2.
  struct Terms { float p, q, dp, dq; };
  auto terms = [&](float a, float b) -> Terms {
    const float P = fmaf(a, k2, -ls2), Q = fmaf(b, k2, -lt2);
    const float hi = fmaxf(P, Q);
    const float e = __builtin_amdgcn_exp2f(fminf(P, Q) - hi);
    const float x = __builtin_amdgcn_exp2f(hi);
    const float lm = hi + __builtin_amdgcn_logf(fmaf(0.5f, e, 0.5f));
    const bool pq = P >= Q;
    return {pq ? x : x * e, pq ? x * e : x, P - lm, Q - lm};
  };
  // loss = 1/2 sum(p (ln p - ln m) + q (ln q - ln m)), sum(p g) with
  // g = 1/2 (ln p - ln m): both summed here without their 1/2 ln 2.
  float loss = 0.0f, gbar = 0.0f;
  auto accumulate = [&](float a, float b) {
    const Terms r = terms(a, b);
    const float pd = r.p * r.dp;
    loss += pd + r.q * r.dq;
    gbar += pd;
  };
  // Pass 2, from the row's end: it starts on the bytes pass 1 fetched last
  // (the likeliest to be still cached), and pass 3 then starts on the bytes
  // this pass fetched last.
  for (int64_t vi = rs.nvec > tid ? tid + (rs.nvec - 1 - tid) / kThreads * kThreads : -1; vi >= 0;
       vi -= kThreads) {
    float a[kVec], b[kVec];
    E::unpack(sv[vi], a);
    E::unpack(tv[vi], b);
#pragma unroll
    for (int i = 0; i < kVec; ++i) accumulate(a[i], b[i]);
  }
  if (tid < rs.head) { float a, b; scalar_at(tid, a, b); accumulate(a, b); }
  if (tid < V - rs.tail0) { float a, b; scalar_at(rs.tail0 + tid, a, b); accumulate(a, b); }
  __syncthreads();
  const float half_ln2 = 0.5f * kLn2;
  const float L = half_ln2 * block_sum<kThreads>(loss, red0);
  const float G2 = block_sum<kThreads>(gbar, red1);
  if (tid == 0) loss_rows[pk.map != nullptr ? static_cast<int64_t>(pk.map[row]) : row] = valid ? L : 0.0f;

  // Pass 3: the student gradient, in place: c p (g - sum(p g)) with c the
  // reduction scale over tau, = c ln2 / 2 p (dP - G2).
  uint4* svw = reinterpret_cast<uint4*>(s + rs.head);
  if (!valid) {
    // The whole row (uniform branch): zeros.
    for (int64_t vi = tid; vi < rs.nvec; vi += kThreads) svw[vi] = make_uint4(0u, 0u, 0u, 0u);
    if (tid < rs.head) E::store(s + tid, 0.0f);
    if (tid < V - rs.tail0) E::store(s + rs.tail0 + tid, 0.0f);
  } else {
    const float c = (grad_shift > 0 ? __builtin_ldexpf(1.0f, grad_shift) : hdr->scale) * inv_tau * half_ln2;
    auto grad = [&](float a, float b) -> float {
      const Terms r = terms(a, b);
      return c * r.p * (r.dp - G2);
    };
    for (int64_t vi = tid; vi < rs.nvec; vi += kThreads) {
      float a[kVec], b[kVec];
      E::unpack(sv[vi], a);
      E::unpack(tv[vi], b);
#pragma unroll
      for (int i = 0; i < kVec; ++i) a[i] = grad(a[i], b[i]);
      svw[vi] = E::pack(a);
    }
    // Scalar head and tail: each lane owns one element, read before it writes.
    if (tid < rs.head) {
      float a, b;
      scalar_at(tid, a, b);
      E::store(s + tid, grad(a, b));
    }
    if (tid < V - rs.tail0) {
      float a, b;
      scalar_at(rs.tail0 + tid, a, b);
      E::store(s + rs.tail0 + tid, grad(a, b));
    }
  }
  if (tid < pad_cols) E::store(s + V + tid, 0.0f);
}

hipError_t launch_row_jsd(int dtype, void* S, const void* Tt, int64_t ld, int64_t rows, int64_t V,
                          int64_t pad_cols, float inv_tau, const int32_t* targets, int32_t ign,
                          const WsHeader* hdr, float* loss_rows, int grad_shift, hipStream_t s,
                          RowPack pk) {
  if (rows <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(rows));
  if (dtype == 1)
    hipLaunchKernelGGL((k_row_jsd<uint16_t, 1024>), grid, dim3(1024), 0, s, static_cast<uint16_t*>(S),
                       static_cast<const uint16_t*>(Tt), ld, V, pad_cols, inv_tau, targets, ign, hdr,
                       loss_rows, grad_shift, pk);
  else if (dtype == 2)
    hipLaunchKernelGGL((k_row_jsd<Half, 1024>), grid, dim3(1024), 0, s, static_cast<Half*>(S),
                       static_cast<const Half*>(Tt), ld, V, pad_cols, inv_tau, targets, ign, hdr,
                       loss_rows, grad_shift, pk);
  else
    hipLaunchKernelGGL((k_row_jsd<float, 1024>), grid, dim3(1024), 0, s, static_cast<float*>(S),
                       static_cast<const float*>(Tt), ld, V, pad_cols, inv_tau, targets, ign, hdr,
                       loss_rows, grad_shift, pk);
  return hipGetLastError();
}

// --------------------------------------------------------------------- DPO

// Sequence log-probabilities: logp[k] = -sum of the CE row losses of rows
// [k * S, (k + 1) * S), in a fixed order (strided lane sums, then a tree).
__global__ __launch_bounds__(256) void k_seq_logp(const float* __restrict__ loss_rows, int64_t S,
                                                  double* __restrict__ logp) {
  __shared__ double part[256];
  const float* r = loss_rows + static_cast<int64_t>(blockIdx.x) * S;
  double acc = 0.0;
  for (int64_t i = threadIdx.x; i < S; i += 256) acc += static_cast<double>(r[i]);
  part[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) logp[blockIdx.x] = -part[0];
}

// Per pair b (chosen sequence b, rejected sequence P + b): the margin
// d = beta ((logp_w - ref_w) - (logp_l - ref_l)), the pair loss softplus(-d),
// their mean, and the per-row gradient factors +-beta sigmoid(-d) / P.
__global__ __launch_bounds__(1024) void k_dpo_pairs(const double* __restrict__ logp,
                                                    const float* __restrict__ ref, int64_t P,
                                                    int64_t S, float beta, float* __restrict__ loss,
                                                    float* __restrict__ pair_loss,
                                                    float* __restrict__ row_scale) {
  __shared__ double part[1024];
  double acc = 0.0;
  for (int64_t b = threadIdx.x; b < P; b += 1024) {
    const double d = static_cast<double>(beta) *
                     ((logp[b] - static_cast<double>(ref[b])) - (logp[P + b] - static_cast<double>(ref[P + b])));
    const double l = d > 0.0 ? log1p(exp(-d)) : -d + log1p(exp(d));   // softplus(-d)
    acc += l;
    if (pair_loss != nullptr) pair_loss[b] = static_cast<float>(l);
  }
  part[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if (threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) loss[0] = P > 0 ? static_cast<float>(part[0] / static_cast<double>(P)) : 0.0f;
  // Row factors, one pair's two sequences per outer step.
  for (int64_t i = threadIdx.x; i < 2 * P * S; i += 1024) {
    const int64_t k = i / S, b = k < P ? k : k - P;
    const double d = static_cast<double>(beta) *
                     ((logp[b] - static_cast<double>(ref[b])) - (logp[P + b] - static_cast<double>(ref[P + b])));
    const double c = static_cast<double>(beta) / (1.0 + exp(d)) / static_cast<double>(P);
    row_scale[i] = static_cast<float>(k < P ? c : -c);
  }
}

hipError_t launch_dpo(const float* loss_rows, int64_t P, int64_t S, const float* ref, float beta,
                      double* logp, float* loss, float* pair_loss, float* row_scale, hipStream_t s) {
  if (P <= 0) return launch_fill_f32(loss, 1, 0.0f, s);
  hipLaunchKernelGGL(k_seq_logp, dim3(static_cast<unsigned>(2 * P)), dim3(256), 0, s, loss_rows, S, logp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_dpo_pairs, dim3(1), dim3(1024), 0, s, logp, ref, P, S, beta, loss, pair_loss,
                     row_scale);
  return hipGetLastError();
}

// ------------------------------------------------------ causal label shift

// targets[b * S + s] = labels[b * S + s + 1] for s < S - 1, ignore_index at
// the last position of each sequence.
__global__ __launch_bounds__(256) void k_shift_labels(const int32_t* __restrict__ labels, int64_t n,
                                                      int64_t S, int32_t ign,
                                                      int32_t* __restrict__ targets) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  targets[i] = (i % S == S - 1) ? ign : labels[i + 1];
}

hipError_t launch_shift_labels(const int32_t* labels, int64_t B, int64_t S, int32_t ign,
                               int32_t* targets, hipStream_t s) {
  const int64_t n = B * S;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_shift_labels, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s,
                     labels, n, S, ign, targets);
  return hipGetLastError();
}

// ------------------------------------------------------------ loss reduce

// Sum of per-row losses in float64, in a fixed order independent of how the
// rows were chunked (lane-strided partial sums over groups of 4 rows, a
// butterfly within each wave, the 16 wave sums in wave order); mean divides
// by the valid-row count. One
// barrier: the launch is latency-bound, so the tree through LDS is kept short.
__global__ __launch_bounds__(1024) void k_reduce_loss(const float* __restrict__ rows, int64_t n,
                                                      const WsHeader* __restrict__ hdr,
                                                      int reduction, float* __restrict__ out) {
  __shared__ double wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // The count, read before the rows through a vector load so that its
  // latency overlaps theirs: read where it is used it added a dependent load
  // after the sum, and a scalar load at the top would be waited for before
  // the rows' loads go out (scalar loads return out of order, so the first
  // use of the kernel arguments waits for all of them).
  const int n_valid = reduction == 2
      ? __builtin_bit_cast(int, __builtin_amdgcn_raw_buffer_load_b32(
            row_rsrc(hdr, sizeof(WsHeader)), static_cast<int>(offsetof(WsHeader, n_valid)), 0, 0))
      : 0;
  double acc = 0.0;
  // 16-byte loads, several in flight per lane, then the unaligned rest.
  const int64_t n4 = (reinterpret_cast<uintptr_t>(rows) & 15u) == 0 ? n / 4 : 0;
  const float4* r4 = reinterpret_cast<const float4*>(rows);
#pragma unroll 8
  for (int64_t i = tid; i < n4; i += 1024) {
    const float4 v = r4[i];
    acc += static_cast<double>(v.x);
    acc += static_cast<double>(v.y);
    acc += static_cast<double>(v.z);
    acc += static_cast<double>(v.w);
  }
  for (int64_t i = n4 * 4 + tid; i < n; i += 1024) acc += static_cast<double>(rows[i]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if (lane == 0) wsum[w] = acc;
  __syncthreads();
  if (tid == 0) {
    double total = 0.0;
#pragma unroll
    for (int k = 0; k < 16; ++k) total += wsum[k];
    if (reduction == 2) total = n_valid > 0 ? total / static_cast<double>(n_valid) : 0.0;
    out[0] = static_cast<float>(total);
  }
}

hipError_t launch_reduce_loss(const float* loss_rows, int64_t n, const WsHeader* hdr, int reduction,
                              float* loss, hipStream_t s) {
  hipLaunchKernelGGL(k_reduce_loss, dim3(1), dim3(1024), 0, s, loss_rows, n, hdr, reduction, loss);
  return hipGetLastError();
}

// ---------------------------------------------------- bias-gradient colsum

// out[v] (+)= f * sum over rows of Z[r, v], f = 2^-out_shift (* *out_scale).
// A workgroup of 4 waves owns a slab of 64 x kVec columns: lane l of every
// wave holds columns [slab + l kVec, + kVec) as one 16-byte vector per row,
// wave w sums rows w, w + 4, w + 8, ... in that order (8 rows' loads in
// flight per lane), and the four waves' sums are added in wave order through
// LDS. The order is fixed, so the sums are deterministic. Z must be 16-byte
// aligned with ldz a multiple of 8 elements (the chunk buffer's layout).
template <typename T, typename TO>
__global__ __launch_bounds__(256) void k_colsum(const T* __restrict__ Z, int64_t ldz, int64_t rows,
                                                int64_t V, TO* __restrict__ out, int accumulate,
                                                const float* __restrict__ out_scale, int out_shift,
                                                const int32_t* __restrict__ live, int64_t live_base) {
  using E = Elem<T>;
  constexpr int kVec = E::kVec;
  __shared__ float part[3][64 * kVec];
  if (live != nullptr) {  // packed chunk: only the live rows
    int64_t n = static_cast<int64_t>(*live) - live_base;
    if (n < 0) n = 0;
    if (n < rows) rows = n;
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t v = (static_cast<int64_t>(blockIdx.x) * 64 + lane) * kVec;
  const bool on = v < V;  // then v + kVec <= ldz: the vector stays inside the row
  float acc[kVec];
#pragma unroll
  for (int e = 0; e < kVec; ++e) acc[e] = 0.0f;
  if (on) {
    const T* p = Z + v;
    int64_t r = w;
    for (; r + 28 < rows; r += 32) {
      uint4 u[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) u[i] = *reinterpret_cast<const uint4*>(p + (r + 4 * i) * ldz);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float f[kVec];
        E::unpack(u[i], f);
#pragma unroll
        for (int e = 0; e < kVec; ++e) acc[e] += f[e];
      }
    }
    for (; r < rows; r += 4) {
      float f[kVec];
      E::unpack(*reinterpret_cast<const uint4*>(p + r * ldz), f);
#pragma unroll
      for (int e = 0; e < kVec; ++e) acc[e] += f[e];
    }
  }
  if (w > 0) {
#pragma unroll
    for (int e = 0; e < kVec; ++e) part[w - 1][lane * kVec + e] = acc[e];
  }
  __syncthreads();
  if (w != 0 || !on) return;
#pragma unroll
  for (int k = 0; k < 3; ++k)
#pragma unroll
    for (int e = 0; e < kVec; ++e) acc[e] += part[k][lane * kVec + e];
  const float f = __builtin_ldexpf(out_scale != nullptr ? *out_scale : 1.0f, -out_shift);
#pragma unroll
  for (int e = 0; e < kVec; ++e) {
    if (v + e >= V) break;
    float val = acc[e] * f;
    if (accumulate) val += Elem<TO>::load(out + v + e);
    Elem<TO>::store(out + v + e, val);
  }
}

template <typename T>
static hipError_t colsum_to(const void* Z, int64_t ldz, int64_t rows, int64_t V, void* out,
                            int out_dtype, bool accumulate, const float* out_scale, int out_shift,
                            RowPack pk, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((V + 64 * Elem<T>::kVec - 1) / (64 * Elem<T>::kVec)));
  const T* z = static_cast<const T*>(Z);
  const int acc = accumulate ? 1 : 0;
  if (out_dtype == 1)
    hipLaunchKernelGGL((k_colsum<T, uint16_t>), grid, dim3(256), 0, s, z, ldz, rows, V,
                       static_cast<uint16_t*>(out), acc, out_scale, out_shift, pk.live, pk.base);
  else if (out_dtype == 2)
    hipLaunchKernelGGL((k_colsum<T, Half>), grid, dim3(256), 0, s, z, ldz, rows, V,
                       static_cast<Half*>(out), acc, out_scale, out_shift, pk.live, pk.base);
  else
    hipLaunchKernelGGL((k_colsum<T, float>), grid, dim3(256), 0, s, z, ldz, rows, V,
                       static_cast<float*>(out), acc, out_scale, out_shift, pk.live, pk.base);
  return hipGetLastError();
}

hipError_t launch_colsum(int dtype, const void* Z, int64_t ldz, int64_t rows, int64_t V, void* out,
                         int out_dtype, bool accumulate, const float* out_scale, int out_shift,
                         hipStream_t s, RowPack pk) {
  if (dtype == 1)
    return colsum_to<uint16_t>(Z, ldz, rows, V, out, out_dtype, accumulate, out_scale, out_shift, pk, s);
  if (dtype == 2)
    return colsum_to<Half>(Z, ldz, rows, V, out, out_dtype, accumulate, out_scale, out_shift, pk, s);
  return colsum_to<float>(Z, ldz, rows, V, out, out_dtype, accumulate, out_scale, out_shift, pk, s);
}

// -------------------------------------------------------- split-K reduce

// out (+)= sum of the K-split partials, splits in index order.
template <typename TO>
__global__ __launch_bounds__(256) void k_splitk_reduce(const float* __restrict__ parts, int splits,
                                                       int64_t stride, int64_t rows, int64_t cols,
                                                       int64_t ld_out, TO* __restrict__ out,
                                                       int accumulate, RowPack pk) {
  if (pk.live != nullptr) {  // packed chunk: only the live rows
    const int64_t n = static_cast<int64_t>(*pk.live) - pk.base;
    if (n < rows) rows = n;
  }
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= rows * cols) return;
  const int64_t r = i / cols, c = i - r * cols;
  float acc = parts[r * cols + c];
  for (int sp = 1; sp < splits; ++sp) acc += parts[sp * stride + r * cols + c];
  const int64_t ro = pk.map != nullptr ? static_cast<int64_t>(pk.map[r]) : r;
  if (accumulate) acc += Elem<TO>::load(out + ro * ld_out + c);
  Elem<TO>::store(out + ro * ld_out + c, acc);
}

// The same, kVec consecutive columns per lane (one 16-byte output vector; the
// same additions in the same order, so the results are identical).
template <typename TO>
__global__ __launch_bounds__(256) void k_splitk_reduce_v(const float* __restrict__ parts, int splits,
                                                         int64_t stride, int64_t rows, int64_t cols,
                                                         int64_t ld_out, TO* __restrict__ out,
                                                         int accumulate, RowPack pk) {
  constexpr int kV = Elem<TO>::kVec;
  if (pk.live != nullptr) {
    const int64_t n = static_cast<int64_t>(*pk.live) - pk.base;
    if (n < rows) rows = n;
  }
  const int64_t cv = cols / kV;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= rows * cv) return;
  const int64_t r = i / cv, c = (i - r * cv) * kV;
  float acc[kV];
#pragma unroll
  for (int q = 0; q < kV; q += 4) {
    const float4 v = *reinterpret_cast<const float4*>(parts + r * cols + c + q);
    acc[q] = v.x; acc[q + 1] = v.y; acc[q + 2] = v.z; acc[q + 3] = v.w;
  }
  for (int sp = 1; sp < splits; ++sp) {
#pragma unroll
    for (int q = 0; q < kV; q += 4) {
      const float4 v = *reinterpret_cast<const float4*>(parts + sp * stride + r * cols + c + q);
      acc[q] += v.x; acc[q + 1] += v.y; acc[q + 2] += v.z; acc[q + 3] += v.w;
    }
  }
  const int64_t ro = pk.map != nullptr ? static_cast<int64_t>(pk.map[r]) : r;
  uint4* o = reinterpret_cast<uint4*>(out + ro * ld_out + c);
  if (accumulate) {
    float old[kV];
    Elem<TO>::unpack(*o, old);
#pragma unroll
    for (int q = 0; q < kV; ++q) acc[q] += old[q];
  }
  *o = Elem<TO>::pack(acc);
}

hipError_t launch_splitk_reduce(const float* parts, int splits, int64_t split_stride, int64_t rows,
                                int64_t cols, int64_t ld_out, void* out, int out_dtype,
                                bool accumulate, hipStream_t s, RowPack pk) {
  const int acc = accumulate ? 1 : 0;
  const int kv = out_dtype == 0 ? 4 : 8;
  if (cols % kv == 0 && ld_out % kv == 0 && split_stride % 4 == 0 &&
      (reinterpret_cast<uintptr_t>(out) & 15u) == 0 && (reinterpret_cast<uintptr_t>(parts) & 15u) == 0) {
    const int64_t nv = rows * (cols / kv);
    const dim3 grid(static_cast<unsigned>((nv + 255) / 256));
    if (out_dtype == 1)
      hipLaunchKernelGGL(k_splitk_reduce_v<uint16_t>, grid, dim3(256), 0, s, parts, splits,
                         split_stride, rows, cols, ld_out, static_cast<uint16_t*>(out), acc, pk);
    else if (out_dtype == 2)
      hipLaunchKernelGGL(k_splitk_reduce_v<Half>, grid, dim3(256), 0, s, parts, splits,
                         split_stride, rows, cols, ld_out, static_cast<Half*>(out), acc, pk);
    else
      hipLaunchKernelGGL(k_splitk_reduce_v<float>, grid, dim3(256), 0, s, parts, splits,
                         split_stride, rows, cols, ld_out, static_cast<float*>(out), acc, pk);
    return hipGetLastError();
  }
  const int64_t n = rows * cols;
  const dim3 grid(static_cast<unsigned>((n + 255) / 256));
  if (out_dtype == 1)
    hipLaunchKernelGGL(k_splitk_reduce<uint16_t>, grid, dim3(256), 0, s, parts, splits, split_stride,
                       rows, cols, ld_out, static_cast<uint16_t*>(out), acc, pk);
  else if (out_dtype == 2)
    hipLaunchKernelGGL(k_splitk_reduce<Half>, grid, dim3(256), 0, s, parts, splits, split_stride,
                       rows, cols, ld_out, static_cast<Half*>(out), acc, pk);
  else
    hipLaunchKernelGGL(k_splitk_reduce<float>, grid, dim3(256), 0, s, parts, splits, split_stride,
                       rows, cols, ld_out, static_cast<float*>(out), acc, pk);
  return hipGetLastError();
}

// -------------------------------------------------------------------- fill

__global__ __launch_bounds__(256) void k_fill_f32(float* __restrict__ p, int64_t n, float v) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * 256)
    p[i] = v;
}

__global__ __launch_bounds__(256) void k_zero16(uint16_t* __restrict__ p, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * 256)
    p[i] = 0;
}

hipError_t launch_zero(void* p, int64_t n, int out_dtype, hipStream_t s) {
  if (out_dtype == 0) return launch_fill_f32(static_cast<float*>(p), n, 0.0f, s);
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_zero16, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     static_cast<uint16_t*>(p), n);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_fill_f32, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

// ------------------------------------------------------------ row packing
//
// A row whose target is ignore_index (or outside [0, V), flagged as an
// error and treated as ignored) has zero loss and a zero dlogits row, so it
// adds nothing to grad_W or grad_bias and its grad_X row is zero. The chunk
// loop can therefore run the three products and the row kernel over the other
// rows only. The list is built in three launches (block counts, their
// exclusive scan, the writes) and keeps the rows in ascending order, so every
// result is deterministic.

constexpr int kPackThreads = 1024, kPackPer = 4;
constexpr int64_t kPackRows = kPackThreads * kPackPer;

int64_t pack_block_count(int64_t n) { return (n + kPackRows - 1) / kPackRows; }

__device__ __forceinline__ bool packed_target(int32_t y, int32_t ign, int64_t V) {
  return y != ign && y >= 0 && static_cast<int64_t>(y) < V;
}

// Exclusive prefix of v over the 1024 lanes of the block (lane order) and the
// block total. wsum holds 16 ints; the caller syncs before reusing it.
__device__ __forceinline__ int block_exclusive_scan(int v, int* wsum, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kPackThreads / 64; ++i) {
    const int t = wsum[i];
    base += i < w ? t : 0;
    tot += t;
  }
  total = tot;
  return base + x - v;
}

__global__ __launch_bounds__(kPackThreads) void k_pack_count(const int32_t* __restrict__ t,
                                                             int64_t n, int64_t V, int32_t ign,
                                                             int32_t* __restrict__ counts) {
  __shared__ int wsum[kPackThreads / 64];
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * kPackRows + threadIdx.x * kPackPer;
  int c = 0;
#pragma unroll
  for (int i = 0; i < kPackPer; ++i)
    if (r0 + i < n && packed_target(t[r0 + i], ign, V)) ++c;
  int total;
  block_exclusive_scan(c, wsum, total);
  if (threadIdx.x == 0) counts[blockIdx.x] = total;
}

// counts[b] := rows packed by blocks before b; hdr->n_packed := all of them.
__global__ __launch_bounds__(kPackThreads) void k_pack_scan(int32_t* __restrict__ counts,
                                                            int64_t nb, WsHeader* __restrict__ hdr) {
  __shared__ int wsum[kPackThreads / 64];
  int carry = 0;
  for (int64_t b0 = 0; b0 < nb; b0 += kPackThreads) {
    const int64_t b = b0 + threadIdx.x;
    const int v = b < nb ? counts[b] : 0;
    int total;
    const int ex = block_exclusive_scan(v, wsum, total);
    if (b < nb) counts[b] = carry + ex;
    carry += total;
    __syncthreads();  // wsum is rewritten by the next round
  }
  if (threadIdx.x == 0) hdr->n_packed = carry;
}

__global__ __launch_bounds__(kPackThreads) void k_pack_write(const int32_t* __restrict__ t,
                                                             int64_t n, int64_t V, int32_t ign,
                                                             const int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ map,
                                                             int32_t* __restrict__ packed,
                                                             float* __restrict__ loss_rows) {
  __shared__ int wsum[kPackThreads / 64];
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * kPackRows + threadIdx.x * kPackPer;
  int32_t y[kPackPer];
  int c = 0;
#pragma unroll
  for (int i = 0; i < kPackPer; ++i) {
    y[i] = r0 + i < n ? t[r0 + i] : ign;
    c += packed_target(y[i], ign, V) ? 1 : 0;
  }
  int total;
  int64_t pos = static_cast<int64_t>(offsets[blockIdx.x]) + block_exclusive_scan(c, wsum, total);
#pragma unroll
  for (int i = 0; i < kPackPer; ++i) {
    const int64_t r = r0 + i;
    if (r >= n) break;
    if (packed_target(y[i], ign, V)) {
      map[pos] = static_cast<int32_t>(r);
      packed[pos] = y[i];
      ++pos;
    } else if (loss_rows != nullptr) {
      loss_rows[r] = 0.0f;
    }
  }
}

hipError_t launch_pack_rows(const int32_t* targets, int64_t n, int64_t V, int32_t ign,
                            int32_t* map, int32_t* packed_targets, int32_t* block_counts,
                            WsHeader* hdr, float* loss_rows, hipStream_t s) {
  const int64_t nb = pack_block_count(n);
  if (nb > 0) {
    hipLaunchKernelGGL(k_pack_count, dim3(static_cast<unsigned>(nb)), dim3(kPackThreads), 0, s,
                       targets, n, V, ign, block_counts);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_pack_scan, dim3(1), dim3(kPackThreads), 0, s, block_counts, nb, hdr);
  if (nb == 0) return hipGetLastError();
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_pack_write, dim3(static_cast<unsigned>(nb)), dim3(kPackThreads), 0, s,
                     targets, n, V, ign, block_counts, map, packed_targets, loss_rows);
  return hipGetLastError();
}

// One workgroup per chunk row; 16-byte copies.
__global__ __launch_bounds__(256) void k_gather_rows(const uint4* __restrict__ src, int64_t vecs,
                                                     RowPack pk, uint4* __restrict__ out) {
  const int64_t r = blockIdx.x;
  if (r >= static_cast<int64_t>(*pk.live) - pk.base) return;
  const uint4* a = src + static_cast<int64_t>(pk.map[r]) * vecs;
  uint4* b = out + r * vecs;
  for (int64_t v = threadIdx.x; v < vecs; v += 256) b[v] = a[v];
}

hipError_t launch_gather_rows(const void* src, int64_t row_bytes, int64_t rows, RowPack pk,
                              void* out, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (row_bytes % 16 != 0 || pk.live == nullptr || pk.map == nullptr) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_gather_rows, dim3(static_cast<unsigned>(rows)), dim3(256), 0, s,
                     static_cast<const uint4*>(src), row_bytes / 16, pk, static_cast<uint4*>(out));
  return hipGetLastError();
}

// Tiles of 64 chunk rows x 64 columns (16-bit elements): the live rows are
// read once, stored row-major to out ([rows, H]) and, through LDS, transposed
// to out_t ([H, ldt], columns = chunk rows; the tile's rows past the live
// count are written as zeros).
__global__ __launch_bounds__(256) void k_gather_rows_t(const uint16_t* __restrict__ src, int64_t H,
                                                       RowPack pk, uint16_t* __restrict__ out,
                                                       uint16_t* __restrict__ out_t, int64_t ldt) {
  __shared__ __align__(16) uint16_t tile[64][72];  // [row][column]
  const int64_t live = static_cast<int64_t>(*pk.live) - pk.base;
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * 64, h0 = static_cast<int64_t>(blockIdx.y) * 64;
  if (r0 >= live) return;
  const int t = threadIdx.x;
#pragma unroll
  for (int i = t; i < 512; i += 256) {
    const int r = i >> 3, c = i & 7;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (r0 + r < live && h0 + c * 8 < H) {
      v = *reinterpret_cast<const uint4*>(src + static_cast<int64_t>(pk.map[r0 + r]) * H + h0 + c * 8);
      *reinterpret_cast<uint4*>(out + (r0 + r) * H + h0 + c * 8) = v;
    }
    *reinterpret_cast<uint4*>(&tile[r][c * 8]) = v;
  }
  __syncthreads();
#pragma unroll
  for (int i = t; i < 512; i += 256) {
    const int hh = i >> 3, c = i & 7;
    if (h0 + hh >= H) continue;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = static_cast<uint32_t>(tile[c * 8 + 2 * e][hh]) |
             (static_cast<uint32_t>(tile[c * 8 + 2 * e + 1][hh]) << 16);
    *reinterpret_cast<uint4*>(out_t + (h0 + hh) * ldt + r0 + c * 8) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

hipError_t launch_gather_rows_t(const void* src, int64_t H, int64_t rows, RowPack pk, void* out,
                                void* out_t, int64_t ldt, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (H % 8 != 0 || ldt % 64 != 0 || ldt < rows || pk.live == nullptr || pk.map == nullptr)
    return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>((rows + 63) / 64), static_cast<unsigned>((H + 63) / 64));
  hipLaunchKernelGGL(k_gather_rows_t, grid, dim3(256), 0, s, static_cast<const uint16_t*>(src), H, pk,
                     static_cast<uint16_t*>(out), static_cast<uint16_t*>(out_t), ldt);
  return hipGetLastError();
}

// Workgroups stride over the rows (the grid is capped, so any n launches).
__global__ __launch_bounds__(256) void k_zero_dead_rows(const int32_t* __restrict__ t, int64_t n,
                                                        int64_t V, int32_t ign,
                                                        uint4* __restrict__ G, int64_t vecs) {
  for (int64_t r = blockIdx.x; r < n; r += gridDim.x) {
    if (packed_target(t[r], ign, V)) continue;
    uint4* g = G + r * vecs;
    for (int64_t v = threadIdx.x; v < vecs; v += 256) g[v] = make_uint4(0u, 0u, 0u, 0u);
  }
}

hipError_t launch_zero_dead_rows(const int32_t* targets, int64_t n, int64_t V, int32_t ign,
                                 void* G, int64_t row_bytes, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (row_bytes % 16 != 0) return hipErrorInvalidValue;
  const int64_t blocks = n < 65536 ? n : 65536;
  hipLaunchKernelGGL(k_zero_dead_rows, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     targets, n, V, ign, static_cast<uint4*>(G), row_bytes / 16);
  return hipGetLastError();
}

}  // namespace lce
