// The three dense contractions of FLCE (torchtune + Liger blog, Figure 1 text:
// the head projection of each row chunk, then the chunk's hidden-state
// gradient and the accumulated head gradient):
//   logits   Z_c  = X_c W^T (+ b)   A = X_c  (k-major)  B = W  (k-major)
//   grad_X   dX_c = dZ_c W          A = dZ_c (k-major)  B = W  (n-major)
//   grad_W   dW  += dZ_c^T X_c      A = dZ_c (m-major)  B = X_c^T gathered
//                                   (k-major), or X_c as stored (n-major)
//
// 16-bit path: v_mfma_f32_32x32x16_bf16 (or _f16 for IEEE half inputs, the
// DeepSpeed vocab-parallel CE page's FP16 case) with fp32 accumulation,
// 256x256 tiles on 4 waves, operands staged in LDS by direct HBM->LDS loads,
// K in 64-wide steps through a ring of five single-operand slots (namespace
// mfma2::ring; see the comment there).
// fp32 path: a plain LDS-tiled VALU kernel (namespace valu).
#include "lce_common.h"

namespace lce {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

namespace tiles {

#ifndef LCE_GROUP_M
#define LCE_GROUP_M 4
#endif
constexpr int kGroupM = LCE_GROUP_M;  // m-tiles per group in the tile order

// Linear workgroup id -> (split, m-tile, n-tile). Workgroups are dealt to
// the 8 XCDs round-robin, so ids are first regrouped so that each XCD gets a
// contiguous range of tiles; inside it, groups of kGroupM m-tiles are swept
// along n so that concurrently running tiles share A and B panels in that
// XCD's L2.
__device__ __forceinline__ void tile_of(int64_t bid, int64_t tiles_m, int64_t tiles_n, int splits,
                                        int64_t& tm, int64_t& tn, int& sp) {
  const int64_t total = tiles_m * tiles_n * splits;
  const int64_t q = total / 8, rem = total % 8;
  const int64_t xcd = bid % 8, slot = bid / 8;
  int64_t id = xcd < rem ? xcd * (q + 1) + slot : rem * (q + 1) + (xcd - rem) * q + slot;
  sp = static_cast<int>(id % splits);
  id /= splits;
  const int64_t per_group = kGroupM * tiles_n;
  const int64_t g = id / per_group;
  const int64_t first_m = g * kGroupM;
  int64_t gsize = tiles_m - first_m;
  if (gsize > kGroupM) gsize = kGroupM;
  const int64_t in_g = id - g * per_group;
  tm = first_m + in_g % gsize;
  tn = in_g / gsize;
}

}  // namespace tiles

// Row packing: the extent of M or K that exists for this call, read on the
// device (the host launches the grid for the largest possible chunk). A
// shorter M also shortens the tile list: the live tiles are renumbered from
// workgroup 0, so they are dealt over all eight XCDs as a full grid's are,
// and the workgroups past them exit. Returns false for those.
__device__ __forceinline__ bool apply_live(GemmDesc& d, int64_t& tiles_m, int64_t tiles_n, int bm,
                                           int64_t bid) {
  if (d.live == nullptr) return true;
  int64_t n = static_cast<int64_t>(*d.live) - d.live_base;
  if (n < 0) n = 0;
  if (d.live_dim == 0) {
    if (n < d.M) d.M = n;
    tiles_m = (d.M + bm - 1) / bm;
    return bid < tiles_m * tiles_n * d.k_splits;
  }
  if (n < d.K) d.K = n;
  return true;
}

// ---------------------------------------------------------------------------
// MFMA GEMMs for 16-bit inputs (bf16 / fp16, fp32 accumulation).
//
// Operand tiles reach LDS through buffer_load_dwordx4 ... lds: the data never
// passes through registers, and rows past the operand's end and K-tails read
// as zero through the buffer descriptor's range check instead of branches.
// Operands that are k-contiguous in HBM are stored [row][k] and read with
// ds_read_b128; m/n-contiguous operands are stored [k][mn] as loaded and read
// with ds_read_b64_tr_b16, which hands each lane four consecutive k of one
// column. Both layouts XOR-swizzle their 16-byte slots so the MFMA operand
// reads are bank-conflict free.
// Non-temporal output stores (out_store): 0.2-0.3% per FLCE step in
// alternating same-box runs; 0 gives plain stores.
#ifndef LCE_NT_STORES
#define LCE_NT_STORES 1
#endif

namespace mfma2 {

constexpr int kBM = 256;                      // output tile: 256 x 256
constexpr int kOOB = 0x7FFFFFF0;              // buffer offset that reads as zero

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4_t lds_v4;

// Wave index as a scalar (the compiler cannot see that threadIdx.x >> 6 is
// uniform across a wave).
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ int mswz(int k) {
  const int i = k & 3;
  return ((i & 1) << 1) | ((i & 2) << 1) | ((i & 1) << 3);
}
// Element offset of (k, mn) in an mn-major tile [k][256].
__device__ __forceinline__ int moff(int k, int mn) {
  return k * kBM + (((mn >> 3) ^ mswz(k)) << 3) + (mn & 7);
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer descriptor over [base, base + bytes) in scalar registers; reads
// past the end return zero.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes <= 0 ? 0 : (bytes >= 0x7FFFFFFF ? 0x7FFFFFFF : static_cast<int>(bytes));
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(a)));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(a >> 32)));
  void* p = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, static_cast<short>(0),
                                           __builtin_amdgcn_readfirstlane(n), 0x00020000);
}

// 16 bytes per lane from buffer offset voff to LDS dst + 16 * lane.
__device__ __forceinline__ void dma16(rsrc_t r, uint16_t* dst, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, voff, 0, 0, 0);
}

template <int kN>
__device__ __forceinline__ void wait_vmcnt() {
  // vmcnt = kN; expcnt and lgkmcnt at their maxima (not waited on).
  __builtin_amdgcn_s_waitcnt((kN & 15) | ((kN >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
}
__device__ __forceinline__ void block_sync() {
  __builtin_amdgcn_sched_barrier(0);
  wait_lgkm0();
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// A wave's fragments for one 16-wide k step: 4 blocks of 32 rows of A and
// kFJ blocks of 32 columns of B.
template <int kFJ>
struct Frags {
  bf16x8_t a[4], b[kFJ];
};

// Output through LDS. The MFMA result layout gives each lane 4 consecutive
// columns of one row, so direct stores touch 32 rows per instruction with 8
// or 16 bytes each. Each wave instead takes its result 128 x 64 at a time,
// writes part of that (64 rows for bf16, 32 for fp32) into its own LDS
// region and reads it back as whole row segments: 8 lanes per 128-byte row
// (bf16) or 16 lanes per 256-byte row (fp32), so every store instruction
// covers full cache lines. Slots are XOR-swizzled by row to spread the
// column-wise writes over the banks.

// Output stores. With LCE_NT_STORES they are non-temporal: the outputs
// (chunk logits, gradients) are not read again by this kernel, so they are
// kept from displacing the operand panels that other tiles still read.
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
template <typename V>
__device__ __forceinline__ void out_store(V* p, const V& v) {
#if LCE_NT_STORES
  static_assert(sizeof(V) == 8 || sizeof(V) == 16, "8- or 16-byte stores");
  if constexpr (sizeof(V) == 16)
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, v), reinterpret_cast<u32x4_t*>(p));
  else
    __builtin_nontemporal_store(__builtin_bit_cast(u32x2_t, v), reinterpret_cast<u32x2_t*>(p));
#else
  *p = v;
#endif
}

// Lanes of one wave exchange data through LDS: LDS executes a wave's
// instructions in order, so only the compiler must not reorder.
__device__ __forceinline__ void wave_lds_fence() {
  wait_lgkm0();
  __builtin_amdgcn_wave_barrier();
}

// 16-bit logits (+ bias): kTy 0 bf16, 1 fp16.
template <int kTy, int kFJ>
__device__ __forceinline__ void epilogue_16(const f32x16_t (&acc)[4][kFJ], const GemmDesc& d,
                                              int64_t m0, int64_t n0, int row0, int col0, char* reg) {
  static_assert(kFJ == 2, "64 output columns per wave");
  const int lane = threadIdx.x & 63, l32 = lane & 31, lhi = lane >> 5;
  const uint16_t* bias = static_cast<const uint16_t*>(d.bias);
  // The lane's bias values: 4 consecutive columns for each (j, q), the same
  // for every row, loaded once: as 8-byte vectors when the bias is 8-byte
  // aligned (n is a multiple of 4), else, and at the end of the row,
  // element by element.
  float bv[kFJ][4][4];
#pragma unroll
  for (int j = 0; j < kFJ; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) bv[j][q][e] = 0.0f;
  if (bias != nullptr) {
    auto to_f32 = [](uint16_t h) { return kTy == 1 ? f16_to_f32(h) : bf16_to_f32(h); };
#pragma unroll
    for (int j = 0; j < kFJ; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t n = n0 + col0 + j * 32 + q * 8 + lhi * 4;
        if (n + 3 < d.N && (reinterpret_cast<uintptr_t>(bias) & 7u) == 0) {
          const uint2 w = *reinterpret_cast<const uint2*>(bias + n);
          bv[j][q][0] = to_f32(static_cast<uint16_t>(w.x));
          bv[j][q][1] = to_f32(static_cast<uint16_t>(w.x >> 16));
          bv[j][q][2] = to_f32(static_cast<uint16_t>(w.y));
          bv[j][q][3] = to_f32(static_cast<uint16_t>(w.y >> 16));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < d.N) bv[j][q][e] = to_f32(bias[n + e]);
        }
      }
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      const int r = ii * 32 + l32;
#pragma unroll
      for (int j = 0; j < kFJ; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x16_t& a = acc[2 * h + ii][j];
          float v[4] = {a[q * 4 + 0] + bv[j][q][0], a[q * 4 + 1] + bv[j][q][1],
                        a[q * 4 + 2] + bv[j][q][2], a[q * 4 + 3] + bv[j][q][3]};
          const int slot = j * 4 + q;
          *reinterpret_cast<uint2*>(reg + r * 128 + ((slot ^ ((r >> 1) & 7)) << 4) + lhi * 8) =
              kTy == 1 ? make_uint2(pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3]))
                       : make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        }
    }
    wave_lds_fence();
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = u * 8 + (lane >> 3), sl = lane & 7;
      const uint4 val = *reinterpret_cast<const uint4*>(reg + r * 128 + ((sl ^ ((r >> 1) & 7)) << 4));
      const int64_t m = m0 + row0 + h * 64 + r;
      const int64_t n = n0 + col0 + sl * 8;
      if (m >= d.M || n >= d.N) continue;
      uint16_t* c = static_cast<uint16_t*>(d.C) + m * d.ldc + n;
      if (n + 7 < d.N) {
        out_store(reinterpret_cast<uint4*>(c), val);
      } else {
        const uint32_t w[4] = {val.x, val.y, val.z, val.w};
        for (int e = 0; e < 8 && n + e < d.N; ++e)
          c[e] = static_cast<uint16_t>(w[e >> 1] >> ((e & 1) * 16));
      }
    }
    wave_lds_fence();
  }
}

template <int kEpi, int kTy, int kFJ>
__device__ __forceinline__ void epilogue_f32(const f32x16_t (&acc)[4][kFJ], const GemmDesc& d,
                                             int64_t m0, int64_t n0, int sp, int row0, int col0,
                                             char* reg) {
  static_assert(kFJ == 2, "64 output columns per wave");
  // fp32 accumulators out as float, or rounded to the 16-bit input type
  // (kTy 0 bf16, 1 fp16); accumulating variants add the old value first.
  constexpr bool k16 = kEpi == kEpiStore16 || kEpi == kEpiAccum16;
  constexpr bool kAcc = kEpi == kEpiAccumF32 || kEpi == kEpiAccum16;
  constexpr int kEb = k16 ? 2 : 4;  // output element bytes
  const int lane = threadIdx.x & 63, l32 = lane & 31, lhi = lane >> 5;
  char* C = static_cast<char*>(d.C) + (static_cast<int64_t>(sp) * d.split_stride) * kEb;
  // Deferred gradient scaling (exact power of two, then the device scale).
  const float f = __builtin_ldexpf(d.out_scale != nullptr ? *d.out_scale : 1.0f, -d.out_shift);
  auto to_f32 = [](uint16_t h) { return kTy == 1 ? f16_to_f32(h) : bf16_to_f32(h); };
  auto pack2 = [](float x, float y) { return kTy == 1 ? pack_f16x2(x, y) : pack_bf16x2(x, y); };
  // A quarter (32 rows) of the wave's result at a time.
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const int64_t mh = m0 + row0 + h * 32;
    // Accumulating: fetch the quarter's old row segments first, in one batch
    // (range-checked buffer loads read zeros outside the matrix), so their
    // latency overlaps the staging through LDS.
    float4 old[8];
    if constexpr (kAcc) {
      const rsrc_t rc = make_rsrc(C + (mh * d.ldc + n0 + col0) * kEb, 32 * d.ldc * kEb);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int r = u * 4 + (lane >> 4), sl = lane & 15;
        const bool ok = mh + r < d.M && n0 + col0 + sl * 4 + 3 < d.N;
        const int voff = ok ? static_cast<int>(r * d.ldc * kEb) + sl * 4 * kEb : kOOB;
        if constexpr (k16) {
          const uint2 w = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rc, voff, 0, 0));
          old[u] = make_float4(to_f32(static_cast<uint16_t>(w.x)), to_f32(static_cast<uint16_t>(w.x >> 16)),
                               to_f32(static_cast<uint16_t>(w.y)), to_f32(static_cast<uint16_t>(w.y >> 16)));
        } else {
          old[u] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rc, voff, 0, 0));
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kFJ; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x16_t& a = acc[h][j];
        const int slot = j * 8 + q * 2 + lhi;
        *reinterpret_cast<float4*>(reg + l32 * 256 + ((slot ^ (l32 & 15)) << 4)) =
            make_float4(a[q * 4 + 0], a[q * 4 + 1], a[q * 4 + 2], a[q * 4 + 3]);
      }
    wave_lds_fence();
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = u * 4 + (lane >> 4), sl = lane & 15;
      float4 o = *reinterpret_cast<const float4*>(reg + r * 256 + ((sl ^ (r & 15)) << 4));
      o.x *= f; o.y *= f; o.z *= f; o.w *= f;
      const int64_t m = mh + r;
      const int64_t n = n0 + col0 + sl * 4;
      if (m >= d.M || n >= d.N) continue;
      // Packed rows go back to their original row (storing epilogues only).
      const int64_t mo = (!kAcc && d.row_map != nullptr) ? static_cast<int64_t>(d.row_map[m]) : m;
      char* c = C + (mo * d.ldc + n) * kEb;
      if (n + 3 < d.N) {
        if constexpr (kAcc) {
          o.x += old[u].x; o.y += old[u].y; o.z += old[u].z; o.w += old[u].w;
        }
        if constexpr (k16)
          out_store(reinterpret_cast<uint2*>(c), make_uint2(pack2(o.x, o.y), pack2(o.z, o.w)));
        else
          out_store(reinterpret_cast<float4*>(c), o);
      } else {
        const float w[4] = {o.x, o.y, o.z, o.w};
        for (int e = 0; e < 4 && n + e < d.N; ++e) {
          if constexpr (k16) {
            uint16_t* c16 = reinterpret_cast<uint16_t*>(c) + e;
            const float v = kAcc ? to_f32(*c16) + w[e] : w[e];
            *c16 = static_cast<uint16_t>(pack2(v, 0.0f) & 0xFFFFu);
          } else {
            float* c32 = reinterpret_cast<float*>(c) + e;
            *c32 = kAcc ? *c32 + w[e] : w[e];
          }
        }
      }
    }
    wave_lds_fence();
  }
}

// ---------------------------------------------------------------------------
// The ring pipeline: 64-wide k steps through five LDS slots of 32 KiB.
//
// Each slot holds one operand of one k step (256 rows x 64 k). With 64-wide
// steps a k-major direct load covers 8 rows x 128 bytes, whole cache lines,
// where a 32-wide stage covers 16 half lines: the texture unit, which limits
// the k-major loads, handles half as many lines per byte. Two full stages of
// 64 KiB would leave only one step of loads in flight; five single-operand
// slots keep three operand loads (96 KiB) in flight while two are read, as
// much as the four 32-wide stages. Loads go out in the order A_0, B_0, A_1,
// B_1, ..., load j into slot j % 5, so step s reads A_s from slot 2s % 5 and
// B_s from slot (2s + 1) % 5. The five slots are five LDS objects and the main
// loop is unrolled by five steps, so every slot index is a compile-time
// constant: the compiler sees which slot each direct load writes and each LDS
// read reads, waits only for the loads a read depends on, and the loads can
// be scheduled between the MFMAs like any other instruction. Used for all
// three products.
//
// k-major slots are [row][64] with the 16-byte chunk c of row r at position
// c ^ rswz(r); mn-major slots are [k][256] with the mn-major swizzle above.
namespace ring {

constexpr int kRK = 64;
constexpr int kSlotElems = kBM * kRK;

__shared__ __align__(16) uint16_t g_slot0[kSlotElems];
__shared__ __align__(16) uint16_t g_slot1[kSlotElems];
__shared__ __align__(16) uint16_t g_slot2[kSlotElems];
__shared__ __align__(16) uint16_t g_slot3[kSlotElems];
__shared__ __align__(16) uint16_t g_slot4[kSlotElems];

template <int kI>
__device__ __forceinline__ uint16_t* slot_buf() {
  if constexpr (kI == 0) return g_slot0;
  else if constexpr (kI == 1) return g_slot1;
  else if constexpr (kI == 2) return g_slot2;
  else if constexpr (kI == 3) return g_slot3;
  else return g_slot4;
}

// Conflict-free ds_read_b128 of 32 consecutive rows at one chunk, for banks
// served 8 or 16 lanes at a time: rows 0..7 and each parity class of rows
// 0..15 map to distinct positions.
__device__ __forceinline__ int rswz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// One operand in the ring: this wave's kInstr of the 32 direct loads of a
// step (kW waves share them; issued in parts, kFirst..kFirst+kCount-1) and
// the MFMA fragment reads.
template <bool kKMajor, int kW>
struct ROp;

template <int kW>
struct ROp<true, kW> {
  static constexpr int kInstr = kBM / 8 / kW;
  static constexpr int kReads = 1;  // LDS reads per fragment
  rsrc_t rsrc;
  int voff0[kInstr], kc8[kInstr];

  __device__ __forceinline__ static int first_row(int w, int t) { return (w * kInstr + t) * 8; }

  __device__ __forceinline__ void init(const uint16_t* P, int64_t ld, int64_t rows, int64_t r0) {
    const int lane = threadIdx.x & 63, w = wave_id();
    int64_t nrows = rows - r0;
    if (nrows > kBM) nrows = kBM;
    rsrc = make_rsrc(P + r0 * ld, nrows * ld * 2);
#pragma unroll
    for (int t = 0; t < kInstr; ++t) {
      const int row = first_row(w, t) + (lane >> 3);
      const int kc = (lane & 7) ^ rswz(row);
      kc8[t] = kc * 8;
      voff0[t] = static_cast<int>(row * ld * 2) + kc * 16;
    }
  }
  template <int kFirst, int kCount>
  __device__ __forceinline__ void issue(uint16_t* dst, int64_t k0, int64_t kend) const {
    const int w = wave_id();
    const int64_t klim = kend - k0;
#pragma unroll
    for (int t = kFirst; t < kFirst + kCount; ++t) {
      const int voff = kc8[t] < klim ? voff0[t] + static_cast<int>(k0 * 2) : kOOB;
      dma16(rsrc, dst + first_row(w, t) * kRK, voff);
    }
  }
  int fbase;  // first row of fragment 0
  __device__ __forceinline__ void frags(int base0) { fbase = base0; }
  // Fragment f: rows fbase + 32 f + lane % 32, k-half lane / 32 of step kk.
  __device__ __forceinline__ bf16x8_t frag(const uint16_t* src, int f, int kk) const {
    const int lane = threadIdx.x & 63, r = lane & 31, c = kk * 2 + (lane >> 5);
    return *reinterpret_cast<const bf16x8_t*>(src + (fbase + f * 32) * kRK + r * kRK +
                                              ((c ^ rswz(r)) << 3));
  }
};

template <int kW>
struct ROp<false, kW> {
  static constexpr int kInstr = kRK / 2 / kW;
  static constexpr int kReads = 2;
  const uint16_t* P;
  int64_t ld, r0;
  int moff0[kInstr];

  __device__ __forceinline__ static int first_k(int w, int t) { return (w * kInstr + t) * 2; }

  __device__ __forceinline__ void init(const uint16_t* P_, int64_t ld_, int64_t, int64_t r0_) {
    P = P_; ld = ld_; r0 = r0_;
    const int lane = threadIdx.x & 63, w = wave_id();
#pragma unroll
    for (int t = 0; t < kInstr; ++t) {
      const int k = first_k(w, t) + (lane >> 5);
      const int c = (lane & 31) ^ mswz(k);
      moff0[t] = static_cast<int>(k * ld * 2) + c * 16;
    }
  }
  template <int kFirst, int kCount>
  __device__ __forceinline__ void issue(uint16_t* dst, int64_t k0, int64_t kend) const {
    const int w = wave_id();
    int64_t nk = kend - k0;
    if (nk > kRK) nk = kRK;
    const rsrc_t r = make_rsrc(P + k0 * ld + r0, (nk * ld - r0) * 2);
#pragma unroll
    for (int t = kFirst; t < kFirst + kCount; ++t) dma16(r, dst + first_k(w, t) * kBM, moff0[t]);
  }
  // Byte offset of this lane's first read for fragment f (rows or columns
  // base0 + 32 f) at kk = 0; the swizzle depends on k mod 4 only, so the
  // other reads of a fragment are this offset plus a constant.
  int foff[4];
  __device__ __forceinline__ void frags(int base0) {
    const int lane = threadIdx.x & 63;
    const int i = (lane & 15) >> 2, q = lane & 3;
    const int k = (lane >> 5) * 8 + i;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      int o = moff(k, base0 + f * 32 + ((lane >> 4) & 1) * 16 + q * 4) * 2;
      // Opaque to the optimiser: each read's address stays "slot + offset +
      // constant". Rebuilt from other reads' addresses, the transposed reads
      // lost the LDS alias scopes that tell the wait-count pass they do not
      // overlap the slot being filled, and every such read then waited for
      // all outstanding direct loads (vmcnt(0)): 960 against 1420 TFLOP/s
      // when the other operand is k-contiguous.
      asm volatile("" : "+v"(o));
      foff[f] = o;
    }
  }
  __device__ __forceinline__ bf16x8_t frag(const uint16_t* src, int f, int kk) const {
    const char* s = reinterpret_cast<const char*>(src) + foff[f] + kk * 16 * kBM * 2;
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(s));
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(s + 4 * kBM * 2));
    const short __attribute__((ext_vector_type(8))) v =
        __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8_t, v);
  }
};

// One 16-wide k sub-step: issue() places kDma direct loads, the next
// fragments are read, and the 4 x kFJ MFMAs run on the current ones,
// interleaved as in mma_step.
template <int kTy, int kDma, bool kAK, bool kBKm, int kW, int kFJ, typename Issue>
__device__ __forceinline__ void sub(f32x16_t (&acc)[4][kFJ], const Frags<kFJ>& f, Frags<kFJ>& nf,
                                    const ROp<kAK, kW>& A, const ROp<kBKm, kW>& B,
                                    const uint16_t* srcA, const uint16_t* srcB, int kk,
                                    Issue&& issue) {
  issue();
#pragma unroll
  for (int i = 0; i < 4; ++i) nf.a[i] = A.frag(srcA, i, kk);
#pragma unroll
  for (int j = 0; j < kFJ; ++j) nf.b[j] = B.frag(srcB, j, kk);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < kFJ; ++j)
      if constexpr (kTy == 1)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, f.b[j]),
                                                           __builtin_bit_cast(f16x8_t, f.a[i]),
                                                           acc[i][j], 0, 0, 0);
      else
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
  constexpr int kMfma = 4 * kFJ;
  constexpr int kReads = 4 * ROp<kAK, kW>::kReads + kFJ * ROp<kBKm, kW>::kReads;
#pragma unroll
  for (int t = 0; t < kMfma; ++t) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (t < kReads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if constexpr (kDma > 0)
      if (t % (kMfma / kDma) == 1) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
  }
  if constexpr (kReads > kMfma) __builtin_amdgcn_sched_group_barrier(0x100, kReads - kMfma, 0);
}

// Step s (kS = s % 5) reads A_s from slot 2s % 5 and B_s from (2s + 1) % 5.
// Its first two k16 sub-steps issue A_{s+2} into the slot B_{s-1} used; the
// barrier before the last sub-step waits for A_{s+1}, B_{s+1} and frees this
// step's slots, and the last sub-step issues B_{s+2} into the slot of A_s.
template <int kTy, int kS, bool kAK, bool kBKm, int kW, int kFJ>
__device__ __forceinline__ void step(f32x16_t (&acc)[4][kFJ], Frags<kFJ>& f0, Frags<kFJ>& f1,
                                     const ROp<kAK, kW>& A, const ROp<kBKm, kW>& B, int64_t k2,
                                     int64_t kend) {
  constexpr int sa = (2 * kS) % 5, sb = (2 * kS + 1) % 5, pb = (2 * kS + 4) % 5;
  constexpr int na = (2 * kS + 2) % 5, nb = (2 * kS + 3) % 5;
  constexpr int kI = ROp<kAK, kW>::kInstr, kH = kI / 2;
  static_assert(kI == ROp<kBKm, kW>::kInstr, "equal load counts per operand");
  const uint16_t* a = slot_buf<sa>();
  const uint16_t* b = slot_buf<sb>();
  sub<kTy, kH, kAK, kBKm, kW>(acc, f0, f1, A, B, a, b, 1,
                              [&] { A.template issue<0, kH>(slot_buf<pb>(), k2, kend); });
  sub<kTy, kH, kAK, kBKm, kW>(acc, f1, f0, A, B, a, b, 2,
                              [&] { A.template issue<kH, kH>(slot_buf<pb>(), k2, kend); });
  sub<kTy, 0, kAK, kBKm, kW>(acc, f0, f1, A, B, a, b, 3, [] {});
  // Only A_{s+2} was issued after B_{s+1}; the count relies on there being
  // no other vector memory instruction in the loop (no spills, checked by
  // the launcher).
  wait_vmcnt<kI>();
  block_sync();
  sub<kTy, kI, kAK, kBKm, kW>(acc, f1, f0, A, B, slot_buf<na>(), slot_buf<nb>(), 0,
                              [&] { B.template issue<0, kI>(slot_buf<sa>(), k2, kend); });
}

// kW = 8: 2 x 4 waves of 128 x 64, two per SIMD. kW = 4: 2 x 2 waves of
// 128 x 128, one per SIMD with the 256 accumulators in AGPRs, a third fewer
// LDS reads per MFMA (logits +1.4 to +2.3% over 8 waves; grad_W 0.7% in
// alternating same-box runs). All three products run on 4 waves.
// One output tile of the ring GEMM, for workgroup `bid` of the product's
// own tile numbering (the whole workgroup takes the same path).
template <bool kAK, bool kBKm, int kEpi, int kTy, int kW>
__device__ __forceinline__ void ring_tile(GemmDesc d, int64_t bid, int64_t tiles_m, int64_t tiles_n,
                                          int64_t k_per_split) {
  constexpr int kFJ = 8 / (kW / 2);  // 32-column MFMA blocks per wave
  constexpr bool kAcc = kEpi == kEpiAccumF32 || kEpi == kEpiAccum16;
  // Whole workgroups leave here, before any barrier.
  if (!apply_live(d, tiles_m, tiles_n, kBM, bid)) return;
  int64_t tm, tn;
  int sp;
  tiles::tile_of(bid, tiles_m, tiles_n, d.k_splits, tm, tn, sp);
  const int64_t m0 = tm * kBM, n0 = tn * kBM;
  const int64_t kbeg = static_cast<int64_t>(sp) * k_per_split;
  int64_t kend = kbeg + k_per_split;
  if (kend > d.K) kend = d.K;
  const int ksteps = kend > kbeg ? static_cast<int>((kend - kbeg + kRK - 1) / kRK) : 0;
  if (kAcc && ksteps == 0) return;  // adds nothing
  constexpr int kI = ROp<kAK, kW>::kInstr;
  ROp<kAK, kW> A;
  ROp<kBKm, kW> B;
  A.init(static_cast<const uint16_t*>(d.A), d.lda, d.M, m0);
  B.init(static_cast<const uint16_t*>(d.B), d.ldb, d.N, n0);
  const int wave = wave_id();
  const int row0 = (wave / (kW / 2)) * 128, col0 = (wave % (kW / 2)) * (kFJ * 32);
  A.frags(row0);
  B.frags(col0);
  f32x16_t acc[4][kFJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < kFJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  // Prologue: A_0, B_0, A_1, B_1 into slots 0..3; step 0 then issues A_2
  // into slot 4. Loads past the end of K read zeros, so every step issues
  // the same loads, and the final steps' look-ahead reads stay in bounds.
  if (ksteps > 0) {
    A.template issue<0, kI>(slot_buf<0>(), kbeg, kend);
    B.template issue<0, kI>(slot_buf<1>(), kbeg, kend);
    A.template issue<0, kI>(slot_buf<2>(), kbeg + kRK, kend);
    B.template issue<0, kI>(slot_buf<3>(), kbeg + kRK, kend);
    wait_vmcnt<2 * kI>();
    block_sync();
    Frags<kFJ> f0, f1;
#pragma unroll
    for (int i = 0; i < 4; ++i) f0.a[i] = A.frag(slot_buf<0>(), i, 0);
#pragma unroll
    for (int j = 0; j < kFJ; ++j) f0.b[j] = B.frag(slot_buf<1>(), j, 0);
    int s = 0;
    for (; s + 5 <= ksteps; s += 5) {
      const int64_t k2 = kbeg + static_cast<int64_t>(s + 2) * kRK;
      step<kTy, 0>(acc, f0, f1, A, B, k2, kend);
      step<kTy, 1>(acc, f0, f1, A, B, k2 + kRK, kend);
      step<kTy, 2>(acc, f0, f1, A, B, k2 + 2 * kRK, kend);
      step<kTy, 3>(acc, f0, f1, A, B, k2 + 3 * kRK, kend);
      step<kTy, 4>(acc, f0, f1, A, B, k2 + 4 * kRK, kend);
    }
    const int64_t k2 = kbeg + static_cast<int64_t>(s + 2) * kRK;
    if (s < ksteps) step<kTy, 0>(acc, f0, f1, A, B, k2, kend);
    if (s + 1 < ksteps) step<kTy, 1>(acc, f0, f1, A, B, k2 + kRK, kend);
    if (s + 2 < ksteps) step<kTy, 2>(acc, f0, f1, A, B, k2 + 2 * kRK, kend);
    if (s + 3 < ksteps) step<kTy, 3>(acc, f0, f1, A, B, k2 + 3 * kRK, kend);
    wait_vmcnt<0>();
  }
  // Every wave is done with the slots; each wave stages its output through
  // 8 KiB of slots 0 and 1, 64 columns at a time.
  block_sync();
  char* reg = reinterpret_cast<char*>(wave < 4 ? g_slot0 : g_slot1) + (wave & 3) * 8192;
#pragma unroll
  for (int hj = 0; hj < kFJ / 2; ++hj) {
    f32x16_t part[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) { part[i][0] = acc[i][2 * hj]; part[i][1] = acc[i][2 * hj + 1]; }
    if constexpr (kEpi == kEpiLogits) epilogue_16<kTy, 2>(part, d, m0, n0, row0, col0 + hj * 64, reg);
    else epilogue_f32<kEpi, kTy, 2>(part, d, m0, n0, sp, row0, col0 + hj * 64, reg);
  }
}

template <bool kAK, bool kBKm, int kEpi, int kTy, int kW>
__global__ __launch_bounds__(64 * kW) __attribute__((amdgpu_waves_per_eu(kW / 4, kW / 4)))
void k_ring(GemmDesc d, int64_t tiles_m, int64_t tiles_n, int64_t k_per_split) {
  ring_tile<kAK, kBKm, kEpi, kTy, kW>(d, blockIdx.x, tiles_m, tiles_n, k_per_split);
}

}  // namespace ring
}  // namespace mfma2

template <bool kAK, bool kBKm, int kEpi, int kTy, int kW>
static hipError_t launch_ring(const GemmDesc& d, hipStream_t s) {
  using namespace mfma2;
  const int64_t tiles_m = (d.M + kBM - 1) / kBM, tiles_n = (d.N + kBM - 1) / kBM;
  const int splits = d.k_splits > 1 ? d.k_splits : 1;
  int64_t k_per = (d.K + splits - 1) / splits;
  k_per = (k_per + ring::kRK - 1) / ring::kRK * ring::kRK;
  auto kern = ring::k_ring<kAK, kBKm, kEpi, kTy, kW>;
  // Spill stores would be counted by the loop's explicit vmcnt waits.
  static int spills = -1;
  if (spills < 0) {
    hipFuncAttributes fa;
    const hipError_t e = hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(kern));
    if (e != hipSuccess) return e;
    spills = fa.localSizeBytes != 0;
  }
  if (spills) return hipErrorInvalidDeviceFunction;
  GemmDesc dd = d;
  dd.k_splits = splits;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(tiles_m * tiles_n * splits)), dim3(64 * kW), 0,
                     s, dd, tiles_m, tiles_n, k_per);
  return hipGetLastError();
}

template <int kTy>
static hipError_t launch_mfma_ty(const GemmDesc& d, hipStream_t s) {
  // The layouts of the FLCE products: logits X W^T (both operands
  // k-contiguous), grad_X dZ W (A k-contiguous, B n-contiguous) and grad_W
  // dZ^T X (A m-contiguous; B the transposed gathered rows, k-contiguous, or
  // X itself, n-contiguous).
  if (d.a_kmajor && d.b_kmajor && d.epilogue == kEpiLogits)
    return launch_ring<true, true, kEpiLogits, kTy, 4>(d, s);
  if (d.a_kmajor && !d.b_kmajor && d.epilogue == kEpiStoreF32)
    return launch_ring<true, false, kEpiStoreF32, kTy, 4>(d, s);
  if (d.a_kmajor && !d.b_kmajor && d.epilogue == kEpiAccumF32)
    return launch_ring<true, false, kEpiAccumF32, kTy, 4>(d, s);
  if (d.a_kmajor && !d.b_kmajor && d.epilogue == kEpiStore16)
    return launch_ring<true, false, kEpiStore16, kTy, 4>(d, s);
  if (d.a_kmajor && !d.b_kmajor && d.epilogue == kEpiAccum16)
    return launch_ring<true, false, kEpiAccum16, kTy, 4>(d, s);
  if (!d.a_kmajor && d.b_kmajor && d.epilogue == kEpiStore16)
    return launch_ring<false, true, kEpiStore16, kTy, 4>(d, s);
  if (!d.a_kmajor && d.b_kmajor && d.epilogue == kEpiAccum16)
    return launch_ring<false, true, kEpiAccum16, kTy, 4>(d, s);
  if (!d.a_kmajor && d.b_kmajor && d.epilogue == kEpiStoreF32)
    return launch_ring<false, true, kEpiStoreF32, kTy, 4>(d, s);
  if (!d.a_kmajor && d.b_kmajor && d.epilogue == kEpiAccumF32)
    return launch_ring<false, true, kEpiAccumF32, kTy, 4>(d, s);
  if (!d.a_kmajor && !d.b_kmajor && d.epilogue == kEpiStore16)
    return launch_ring<false, false, kEpiStore16, kTy, 4>(d, s);
  if (!d.a_kmajor && !d.b_kmajor && d.epilogue == kEpiAccum16)
    return launch_ring<false, false, kEpiAccum16, kTy, 4>(d, s);
  if (!d.a_kmajor && !d.b_kmajor && d.epilogue == kEpiStoreF32)
    return launch_ring<false, false, kEpiStoreF32, kTy, 4>(d, s);
  if (!d.a_kmajor && !d.b_kmajor && d.epilogue == kEpiAccumF32)
    return launch_ring<false, false, kEpiAccumF32, kTy, 4>(d, s);
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_16(const GemmDesc& d, bool f16, hipStream_t s) {
  if (d.M <= 0 || d.N <= 0) return hipSuccess;
  // A row map redirects stored rows; an accumulating epilogue reads its old
  // values as contiguous rows and takes none.
  if (d.row_map != nullptr &&
      (d.epilogue == kEpiLogits || d.epilogue == kEpiAccumF32 || d.epilogue == kEpiAccum16))
    return hipErrorInvalidValue;
  return f16 ? launch_mfma_ty<1>(d, s) : launch_mfma_ty<0>(d, s);
}

// ------------------------------------------------------------- fp32 VALU

namespace valu {

constexpr int kT = 64, kTK = 16;

template <bool kAK, bool kBKm, int kEpi>
__global__ __launch_bounds__(256) void k_gemm_f32(GemmDesc d, int64_t tiles_n, int64_t k_per_split) {
  __shared__ float As[kTK][kT + 4];
  __shared__ float Bs[kTK][kT + 4];
  const int64_t tile = blockIdx.x;
  const int sp = blockIdx.y;
  const int64_t m0 = (tile / tiles_n) * kT, n0 = (tile % tiles_n) * kT;
  const int64_t kbeg = static_cast<int64_t>(sp) * k_per_split;
  int64_t kend = kbeg + k_per_split;
  if (kend > d.K) kend = d.K;
  const float* A = static_cast<const float*>(d.A);
  const float* B = static_cast<const float*>(d.B);
  const int t = threadIdx.x, tx = t & 15, ty = t >> 4;
  float acc[4][4] = {};
  for (int64_t k0 = kbeg; k0 < kend; k0 += kTK) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = t + 256 * u;          // 0..1023 over a 64 x 16 tile
      const int r = e >> 4, kk = e & 15;  // row-of-tile, k
      const int64_t k = k0 + kk;
      const int64_t m = m0 + r, n = n0 + r;
      float av = 0.0f, bv = 0.0f;
      if (m < d.M && k < kend) av = kAK ? A[m * d.lda + k] : A[k * d.lda + m];
      if (n < d.N && k < kend) bv = kBKm ? B[n * d.ldb + k] : B[k * d.ldb + n];
      As[kk][r] = av;
      Bs[kk][r] = bv;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kTK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + ty * 4 + i;
    if (m >= d.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + tx * 4 + j;
      if (n >= d.N) continue;
      float v = acc[i][j];
      if constexpr (kEpi == kEpiLogits) {
        if (d.bias != nullptr) v += static_cast<const float*>(d.bias)[n];
        static_cast<float*>(d.C)[m * d.ldc + n] = v;
      } else {
        v = __builtin_ldexpf(v * (d.out_scale != nullptr ? *d.out_scale : 1.0f), -d.out_shift);
        float* c = static_cast<float*>(d.C) + static_cast<int64_t>(sp) * d.split_stride + m * d.ldc + n;
        *c = (kEpi == kEpiAccumF32) ? *c + v : v;
      }
    }
  }
}

}  // namespace valu

template <bool kAK, bool kBKm, int kEpi>
static hipError_t launch_valu(const GemmDesc& d, hipStream_t s) {
  using namespace valu;
  const int64_t tiles_m = (d.M + kT - 1) / kT, tiles_n = (d.N + kT - 1) / kT;
  const int splits = d.k_splits > 1 ? d.k_splits : 1;
  const int64_t k_per = (d.K + splits - 1) / splits;
  hipLaunchKernelGGL((k_gemm_f32<kAK, kBKm, kEpi>), dim3(static_cast<unsigned>(tiles_m * tiles_n), splits),
                     dim3(256), 0, s, d, tiles_n, k_per);
  return hipGetLastError();
}

hipError_t launch_gemm_f32(const GemmDesc& d, hipStream_t s) {
  if (d.M <= 0 || d.N <= 0) return hipSuccess;
  if (d.live != nullptr || d.row_map != nullptr) return hipErrorInvalidValue;  // 16-bit path only
  if (d.a_kmajor && d.b_kmajor && d.epilogue == kEpiLogits) return launch_valu<true, true, kEpiLogits>(d, s);
  if (d.a_kmajor && !d.b_kmajor && d.epilogue == kEpiStoreF32) return launch_valu<true, false, kEpiStoreF32>(d, s);
  if (d.a_kmajor && !d.b_kmajor && d.epilogue == kEpiAccumF32) return launch_valu<true, false, kEpiAccumF32>(d, s);
  if (!d.a_kmajor && !d.b_kmajor && d.epilogue == kEpiStoreF32) return launch_valu<false, false, kEpiStoreF32>(d, s);
  if (!d.a_kmajor && !d.b_kmajor && d.epilogue == kEpiAccumF32) return launch_valu<false, false, kEpiAccumF32>(d, s);
  return hipErrorInvalidValue;
}

}  // namespace lce
