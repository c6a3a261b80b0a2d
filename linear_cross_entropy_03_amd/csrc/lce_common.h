// Shared device helpers and the internal launch interface of liblce03.
//
// Everything here is gfx950 (CDNA4) code: wave64, DPP and ds_swizzle
// cross-lane moves, v_cvt_pk_bf16_f32 rounding, v_exp_f32 / v_log_f32.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lce {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Workspace header written by the target-count kernel at the start of every
// call and read by the kernels after it.
struct WsHeader {
  int32_t n_bad;    // targets neither ignore_index nor inside [0, V)
  int32_t n_valid;  // rows that contribute to the loss
  float scale;      // gradient factor: 1/n_valid (mean, 0 if none), else 1
  int32_t n_packed; // rows listed by the row-packing kernels (== n_valid)
  int32_t pad[60];
};
static_assert(sizeof(WsHeader) == 256, "header is one 256-byte slot");

// ---------------------------------------------------------------- bf16 bits

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  return static_cast<uint16_t>(pack_bf16x2(x, 0.0f) & 0xFFFFu);
}

// ---------------------------------------------------------------- fp16 bits

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// Storage tag of an IEEE half element (2 bytes, like the bf16 uint16_t).
struct Half {
  uint16_t bits;
};
static_assert(sizeof(Half) == 2, "half storage is 2 bytes");

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}
// Two floats -> packed half pair, round to nearest even.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}

// Element access for the storage types: float, bf16 (uint16_t bits) and
// fp16 (Half).
template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kVec = 4;  // elements per 16-byte vector
  __device__ static float load(const float* p) { return *p; }
  __device__ static void store(float* p, float v) { *p = v; }
  __device__ static void unpack(const uint4& u, float* f) {
    f[0] = __uint_as_float(u.x); f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z); f[3] = __uint_as_float(u.w);
  }
  __device__ static uint4 pack(const float* f) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]),
                      __float_as_uint(f[2]), __float_as_uint(f[3]));
  }
};
template <> struct Elem<uint16_t> {
  static constexpr int kVec = 8;
  __device__ static float load(const uint16_t* p) { return bf16_to_f32(*p); }
  __device__ static void store(uint16_t* p, float v) { *p = f32_to_bf16(v); }
  __device__ static void unpack(const uint4& u, float* f) {
    f[0] = bf16_lo(u.x); f[1] = bf16_hi(u.x); f[2] = bf16_lo(u.y); f[3] = bf16_hi(u.y);
    f[4] = bf16_lo(u.z); f[5] = bf16_hi(u.z); f[6] = bf16_lo(u.w); f[7] = bf16_hi(u.w);
  }
  __device__ static uint4 pack(const float* f) {
    return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                      pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
  }
};

template <> struct Elem<Half> {
  static constexpr int kVec = 8;
  __device__ static float load(const Half* p) { return f16_to_f32(p->bits); }
  __device__ static void store(Half* p, float v) {
    p->bits = static_cast<uint16_t>(pack_f16x2(v, 0.0f) & 0xFFFFu);
  }
  __device__ static void unpack(const uint4& u, float* f) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = f16_to_f32(static_cast<uint16_t>(w[i] & 0xFFFFu));
      f[2 * i + 1] = f16_to_f32(static_cast<uint16_t>(w[i] >> 16));
    }
  }
  __device__ static uint4 pack(const float* f) {
    return make_uint4(pack_f16x2(f[0], f[1]), pack_f16x2(f[2], f[3]),
                      pack_f16x2(f[4], f[5]), pack_f16x2(f[6], f[7]));
  }
};

// ------------------------------------------------------- wave64 reductions
// Butterfly within rows of 16 lanes with DPP, across the two rows of each
// 32-lane half with ds_swizzle, across the halves with readlane. Every lane
// returns the same value; the combination order is fixed, so results are
// deterministic.

template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, false));
}
__device__ __forceinline__ float swz_xor16(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
}
__device__ __forceinline__ float lane_f32(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f32<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f32<0x141>(v));  // row_half_mirror
  v = fmaxf(v, dpp_f32<0x140>(v));  // row_mirror
  v = fmaxf(v, swz_xor16(v));
  return fmaxf(lane_f32(v, 0), lane_f32(v, 32));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x141>(v);
  v += dpp_f32<0x140>(v);
  v += swz_xor16(v);
  return lane_f32(v, 0) + lane_f32(v, 32);
}

// Block-wide reductions; `scratch` holds one float per wave and must not be
// reused by the caller before the next __syncthreads().
template <int kThreads>
__device__ __forceinline__ float block_max(float v, float* scratch) {
  constexpr int kWaves = kThreads / 64;
  v = wave_max(v);
  if (kWaves == 1) return v;
  if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = scratch[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) r = fmaxf(r, scratch[w]);
  return r;
}
template <int kThreads>
__device__ __forceinline__ float block_sum(float v, float* scratch) {
  constexpr int kWaves = kThreads / 64;
  v = wave_sum(v);
  if (kWaves == 1) return v;
  if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = scratch[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) r += scratch[w];
  return r;
}

// ------------------------------------------------- internal launch interface
// Host-side launchers; each returns hipSuccess or the launch error.

enum Epilogue : int {
  kEpiLogits = 0,   // C (input dtype) = acc (+ bias[n]); C is [M, ldc]
  kEpiStoreF32 = 1, // C (float) = acc
  kEpiAccumF32 = 2, // C (float) += acc
  kEpiStore16 = 3,  // C (input dtype) = round(acc)
  kEpiAccum16 = 4   // C (input dtype) = round(C + acc)
};

struct GemmDesc {
  const void* A;   // A[m, k] = a_kmajor ? A[m*lda + k] : A[k*lda + m]
  const void* B;   // B[k, n] = b_kmajor ? B[n*ldb + k] : B[k*ldb + n]
  void* C;         // C[m, n] at C[m*ldc + n]
  const void* bias;  // kEpiLogits only, [N] or null
  int64_t lda, ldb, ldc;
  int64_t M, N, K;
  bool a_kmajor, b_kmajor;
  int epilogue;
  int k_splits;        // >1: split K; split s writes C + s*split_stride (kEpiStoreF32 only)
  int64_t split_stride;
  // fp32 epilogues: the product is multiplied by 2^-out_shift and by *out_scale
  // (when not null) before it is stored or added (deferred gradient scaling).
  const float* out_scale;
  int out_shift;
  // Row packing: when `live` is not null the extent of M (live_dim 0) or of K
  // (live_dim 1) is read on the device as clamp(*live - live_base, 0, M or K);
  // tiles past it exit at once. When `row_map` is not null, output row m of a
  // storing fp32/16-bit epilogue goes to row row_map[m] of C.
  const int32_t* live;
  int64_t live_base;
  int live_dim;
  const int32_t* row_map;
};

// The live rows of a chunk of packed rows: row r of the chunk exists when
// r < *live - base, and its results belong to original row map[r] (map is
// already offset to the chunk). A null `live` means every row exists and a
// null `map` that row r is row r.
struct RowPack {
  const int32_t* map;
  const int32_t* live;
  int64_t base;
};

// fp16 dlogits in the chunk buffer: the row kernels store them times a power
// of two (2^15 for the CE rows, whose factor before the shift is at most 1 in
// magnitude) and without the reduction's scale, and the gradient GEMMs and
// column sums apply scale * 2^-shift in fp32. Stored with the mean's
// 1/N_valid, most probabilities of a 128k vocabulary (~1e-5 before scaling)
// would fall below fp16's normal range (6.1e-5); the one-hot term times 2^15
// stays below fp16's largest finite value.
constexpr int kF16GradShift = 15;

// 16-bit inputs (bf16, or fp16 when f16 is set), fp32 accumulation.
hipError_t launch_gemm_16(const GemmDesc& d, bool f16, hipStream_t s);
hipError_t launch_gemm_f32(const GemmDesc& d, hipStream_t s);


hipError_t launch_count_targets(const int32_t* targets, int64_t n, int64_t V,
                                int32_t ignore_index, int reduction, WsHeader* hdr,
                                hipStream_t s);

// Row CE over `rows` rows of Z (row stride ldz). Row r uses target
// targets[r]; its loss goes to loss_rows[r]. When grad != null, grad row r
// (stride ldg; may alias Z) receives scale * (softmax - onehot), and columns
// [V, V + pad_cols) of it are set to zero.
// row_scale: per-row gradient factors, or nullptr for the reduction's scale.
// grad_shift > 0: the gradient is stored times 2^grad_shift (times row_scale
// when given) and without the reduction's scale, which the consumer applies.
// pk: rows past pk.live are skipped, and row r's loss goes to
// loss_rows[pk.map[r]] and its factor is row_scale[pk.map[r]] (row packing).
hipError_t launch_row_ce(int dtype, const void* Z, int64_t ldz, void* grad, int64_t ldg,
                         int64_t rows, int64_t V, int64_t pad_cols, const int32_t* targets,
                         int32_t ign, const WsHeader* hdr, float* loss_rows,
                         const float* row_scale, int grad_shift, hipStream_t s,
                         RowPack pk = RowPack{nullptr, nullptr, 0});

// Row CE over a whole call of `rows` rows (contiguous, stride V) that also
// counts the targets: fills hdr (n_bad, n_valid, scale) as launch_count_targets
// would, in the same launch (two launches where the persistent row kernel
// applies). For calls with few rows (every workgroup reads all targets).
// Gradient stores are non-temporal (the caller's gradient is not reread).
hipError_t launch_row_ce_counted(int dtype, const void* Z, void* grad, int64_t rows, int64_t V,
                                 const int32_t* targets, int32_t ign, int reduction, WsHeader* hdr,
                                 float* loss_rows, hipStream_t s);

hipError_t launch_shard_stats(int dtype, const void* Z, int64_t ldz, int64_t rows,
                              int64_t V_local, int64_t vocab_start, int64_t V_global,
                              const int32_t* targets, int32_t ignore_index, float* row_max,
                              float* row_sumexp, float* row_target, hipStream_t s);
// Shard statistics over a whole call of `rows` rows (stride V_local) that also
// counts the targets against V_global into hdr (sum reduction), in the same
// launch. For calls with few rows.
hipError_t launch_shard_stats_counted(int dtype, const void* Z, int64_t rows, int64_t V_local,
                                      int64_t vocab_start, int64_t V_global,
                                      const int32_t* targets, int32_t ign, float* row_max,
                                      float* row_sumexp, float* row_target, WsHeader* hdr,
                                      hipStream_t s);

hipError_t launch_shard_grad(int dtype, void* Z, int64_t ldz, int64_t rows, int64_t V_local,
                             int64_t pad_cols, int64_t vocab_start, int64_t V_global,
                             const int32_t* targets, int32_t ign, const float* lse,
                             const WsHeader* hdr, int grad_shift, hipStream_t s,
                             RowPack pk = RowPack{nullptr, nullptr, 0});
hipError_t launch_combine_stats(const float* ms, const float* ss, const float* ts, int64_t P,
                                int64_t N, const int32_t* targets, int32_t ign, int64_t V_global,
                                float* lse, float* loss_rows, hipStream_t s);
hipError_t launch_row_jsd(int dtype, void* S, const void* Tt, int64_t ld, int64_t rows, int64_t V,
                          int64_t pad_cols, float inv_tau, const int32_t* targets, int32_t ign,
                          const WsHeader* hdr, float* loss_rows, int grad_shift, hipStream_t s,
                          RowPack pk = RowPack{nullptr, nullptr, 0});
hipError_t launch_dpo(const float* loss_rows, int64_t P, int64_t S, const float* ref, float beta,
                      double* logp, float* loss, float* pair_loss, float* row_scale, hipStream_t s);
hipError_t launch_shift_labels(const int32_t* labels, int64_t B, int64_t S, int32_t ign,
                               int32_t* targets, hipStream_t s);
hipError_t launch_reduce_loss(const float* loss_rows, int64_t n, const WsHeader* hdr,
                              int reduction, float* loss, hipStream_t s);

// Column sums of Z times 2^-out_shift (and *out_scale when not null) into out
// of out_dtype (0 float, 1 bf16, 2 fp16; accumulation rounds once per call).
// pk.live limits the rows summed (row packing). Z 16-byte aligned, ldz a
// multiple of 8 elements.
hipError_t launch_colsum(int dtype, const void* Z, int64_t ldz, int64_t rows, int64_t V,
                         void* out, int out_dtype, bool accumulate, const float* out_scale,
                         int out_shift, hipStream_t s, RowPack pk = RowPack{nullptr, nullptr, 0});

// out (+)= the sum of the K-split partials; out_dtype 0 float, 1 bf16, 2 fp16
// (16-bit outputs are rounded once, after the fp32 sum).
// pk: only live rows are reduced, row r into out row pk.map[r].
hipError_t launch_splitk_reduce(const float* parts, int splits, int64_t split_stride,
                                int64_t rows, int64_t cols, int64_t ld_out, void* out,
                                int out_dtype, bool accumulate, hipStream_t s,
                                RowPack pk = RowPack{nullptr, nullptr, 0});

// Row packing. Rows whose target is ignore_index (or outside [0, V)) add
// nothing to the loss or to any gradient, so the chunk loop can run over the
// other rows only. launch_pack_rows lists them in ascending order: map[j] =
// original row of packed row j, packed_targets[j] its target, hdr->n_packed
// their count; loss_rows[r] = 0 for every other row r (when loss_rows is not
// null). block_counts needs pack_block_count(n) ints.
int64_t pack_block_count(int64_t n);
hipError_t launch_pack_rows(const int32_t* targets, int64_t n, int64_t V, int32_t ign,
                            int32_t* map, int32_t* packed_targets, int32_t* block_counts,
                            WsHeader* hdr, float* loss_rows, hipStream_t s);
// out[r, :] = src[pk.map[r], :] for the live rows r < rows of a chunk; rows
// of row_bytes bytes (a multiple of 16, 16-byte aligned).
hipError_t launch_gather_rows(const void* src, int64_t row_bytes, int64_t rows, RowPack pk,
                              void* out, hipStream_t s);
// The same for 16-bit rows of H elements (H a multiple of 8), also writing
// the transpose: out_t[h, r] = src[pk.map[r], h] ([H, ldt], ldt a multiple of
// 64 and at least rows); columns r of the last 64-row tile past the live
// count are zeros.
hipError_t launch_gather_rows_t(const void* src, int64_t H, int64_t rows, RowPack pk, void* out,
                                void* out_t, int64_t ldt, hipStream_t s);
// Zeros the rows r of G ([n, row_bytes]) whose target is not packed.
hipError_t launch_zero_dead_rows(const int32_t* targets, int64_t n, int64_t V, int32_t ign,
                                 void* G, int64_t row_bytes, hipStream_t s);

hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t s);
// Zeros n elements of out_dtype (0 float, 1 bf16, 2 fp16).
hipError_t launch_zero(void* p, int64_t n, int out_dtype, hipStream_t s);

}  // namespace lce
