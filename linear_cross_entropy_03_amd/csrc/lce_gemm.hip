// The three dense contractions of FLCE (torchtune + Liger blog, Figure 1 text:
// the head projection of each row chunk, then the chunk's hidden-state
// gradient and the accumulated head gradient):
//   logits   Z_c  = X_c W^T (+ b)   A = X_c  (k-major)  B = W  (k-major)
//   grad_X   dX_c = dZ_c W          A = dZ_c (k-major)  B = W  (n-major)
//   grad_W   dW  += dZ_c^T X_c      A = dZ_c (m-major)  B = X_c (n-major)
//
// bf16 path: one MFMA kernel for all three, v_mfma_f32_32x32x16_bf16 with
// fp32 accumulation. A 256x256 output tile per 256-lane workgroup (four
// waves, 128x128 each as 4x4 MFMA blocks), K staged through LDS in steps of
// 64 with two LDS buffers and register prefetch of the next step. Both
// operands are held in LDS k-contiguous, so every MFMA operand is one 16-byte
// LDS read; operands stored m- or n-contiguous in HBM are transposed in
// registers (8x8 bf16 blocks with v_perm_b32) on their way into LDS. LDS
// rows are 128 bytes with an XOR swizzle of the 16-byte slots so that both
// the transposing stores and the MFMA operand reads are bank-conflict free.
//
// fp32 path: a plain LDS-tiled VALU kernel (used for fp32 inputs).
#include "lce_common.h"

namespace lce {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

namespace mfma {

constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kThreads = 256;
constexpr int kTileElems = kBM * kBK;  // per operand per stage (kBM == kBN)
constexpr int kGroupM = 8;             // m-tiles per group in the tile order

// 16-byte slot of (row, k-chunk) inside a 128-byte LDS row.
__device__ __forceinline__ int lds_off(int row, int kc) {
  return row * kBK + ((kc ^ ((row ^ (row >> 3)) & 7)) << 3);
}

// Pick element c of the packed pairs a (k even) and b (k odd), as a pair.
__device__ __forceinline__ uint32_t pick_pair(uint32_t a, uint32_t b, int hi) {
  return __builtin_amdgcn_perm(b, a, hi ? 0x07060302u : 0x05040100u);
}

// in[r]: 8 consecutive mn-values at k = r. out[c]: 8 consecutive k-values at mn = c.
__device__ __forceinline__ void transpose8x8(const uint4 (&in)[8], uint4 (&out)[8]) {
  uint32_t w[8][4];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    w[r][0] = in[r].x; w[r][1] = in[r].y; w[r][2] = in[r].z; w[r][3] = in[r].w;
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    out[c].x = pick_pair(w[0][c >> 1], w[1][c >> 1], c & 1);
    out[c].y = pick_pair(w[2][c >> 1], w[3][c >> 1], c & 1);
    out[c].z = pick_pair(w[4][c >> 1], w[5][c >> 1], c & 1);
    out[c].w = pick_pair(w[6][c >> 1], w[7][c >> 1], c & 1);
  }
}

// One operand's tile [256 rows (m or n)] x [64 k] for one K step.
//  k-major:  lane t loads 16-byte chunks (row t/8 + 32 j, k-chunk t%8), j < 8.
//  mn-major: lane t loads the 8x8 block (k-block t/32, mn-block t%32): eight
//            16-byte rows along mn, transposed before the LDS store.
template <bool kKMajor>
struct TileLoader {
  uint4 r[8];

  __device__ __forceinline__ void load(const uint16_t* __restrict__ P, int64_t ld, int64_t row0,
                                       int64_t rows, int64_t k0, int64_t kbound) {
    const int t = threadIdx.x;
    if constexpr (kKMajor) {
      const int kc = t & 7;
      const int64_t k = k0 + kc * 8;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t row = row0 + (t >> 3) + 32 * j;
        if (row < rows && k < kbound)
          r[j] = *reinterpret_cast<const uint4*>(P + row * ld + k);
        else
          r[j] = make_uint4(0u, 0u, 0u, 0u);
      }
    } else {
      const int64_t mn = row0 + (t & 31) * 8;
      const int64_t kb = k0 + (t >> 5) * 8;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t k = kb + j;
        if (mn < rows && k < kbound)
          r[j] = *reinterpret_cast<const uint4*>(P + k * ld + mn);
        else
          r[j] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  }

  __device__ __forceinline__ void store(uint16_t* lds) const {
    const int t = threadIdx.x;
    if constexpr (kKMajor) {
      const int kc = t & 7;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int row = (t >> 3) + 32 * j;
        *reinterpret_cast<uint4*>(lds + lds_off(row, kc)) = r[j];
      }
    } else {
      uint4 o[8];
      transpose8x8(r, o);
      const int kc = t >> 5;
      const int rb = (t & 31) * 8;
#pragma unroll
      for (int c = 0; c < 8; ++c) *reinterpret_cast<uint4*>(lds + lds_off(rb + c, kc)) = o[c];
    }
  }
};

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

template <bool kAK, bool kBKm, int kEpi>
__global__ __launch_bounds__(kThreads, 1) void k_gemm(GemmDesc d, int64_t tiles_m, int64_t tiles_n,
                                                      int64_t k_per_split) {
  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* As = smem;                      // [2][256][64]
  uint16_t* Bs = smem + 2 * kTileElems;     // [2][256][64]

  int64_t tm, tn;
  int sp;
  tile_of(blockIdx.x, tiles_m, tiles_n, d.k_splits, tm, tn, sp);
  const int64_t m0 = tm * kBM, n0 = tn * kBN;
  const int64_t kbeg = static_cast<int64_t>(sp) * k_per_split;
  int64_t kend = kbeg + k_per_split;
  if (kend > d.K) kend = d.K;
  const int64_t ksteps = kend > kbeg ? (kend - kbeg + kBK - 1) / kBK : 0;

  const uint16_t* A = static_cast<const uint16_t*>(d.A);
  const uint16_t* B = static_cast<const uint16_t*>(d.B);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, lhi = lane >> 5;

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  TileLoader<kAK> la;
  TileLoader<kBKm> lb;
  if (ksteps > 0) {
    la.load(A, d.lda, m0, d.M, kbeg, kend);
    lb.load(B, d.ldb, n0, d.N, kbeg, kend);
    la.store(As);
    lb.store(Bs);
    if (ksteps > 1) {
      la.load(A, d.lda, m0, d.M, kbeg + kBK, kend);
      lb.load(B, d.ldb, n0, d.N, kbeg + kBK, kend);
    }
  }
  __syncthreads();

  for (int64_t ks = 0; ks < ksteps; ++ks) {
    const int cur = static_cast<int>(ks & 1);
    if (ks + 1 < ksteps) {
      la.store(As + (cur ^ 1) * kTileElems);
      lb.store(Bs + (cur ^ 1) * kTileElems);
    }
    if (ks + 2 < ksteps) {
      la.load(A, d.lda, m0, d.M, kbeg + (ks + 2) * kBK, kend);
      lb.load(B, d.ldb, n0, d.N, kbeg + (ks + 2) * kBK, kend);
    }
    const uint16_t* as = As + cur * kTileElems;
    const uint16_t* bs = Bs + cur * kTileElems;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int kc = kk * 2 + lhi;
      bf16x8_t af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(as + lds_off(wm * 128 + i * 32 + l32, kc));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(bs + lds_off(wn * 128 + j * 32 + l32, kc));
      // Operands swapped (B first) so the 32x32 result block is C^T: each
      // lane then holds 4 consecutive n of one m, i.e. contiguous stores.
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }

  // Epilogue. acc[i][j][q*4 + e] is C[m][n] with
  //   m = m0 + wm*128 + i*32 + l32,  n = n0 + wn*128 + j*32 + q*8 + lhi*4 + e.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + wm * 128 + i * 32 + l32;
    if (m >= d.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t n = n0 + wn * 128 + j * 32 + q * 8 + lhi * 4;
        if (n >= d.N) continue;
        float v[4] = {acc[i][j][q * 4 + 0], acc[i][j][q * 4 + 1], acc[i][j][q * 4 + 2],
                      acc[i][j][q * 4 + 3]};
        const bool full = n + 3 < d.N;
        if constexpr (kEpi == kEpiLogits) {
          if (d.bias != nullptr) {
            const uint16_t* b = static_cast<const uint16_t*>(d.bias);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (n + e < d.N) v[e] += bf16_to_f32(b[n + e]);
          }
          uint16_t* c = static_cast<uint16_t*>(d.C) + m * d.ldc + n;
          if (full) {
            *reinterpret_cast<uint2*>(c) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (n + e < d.N) c[e] = f32_to_bf16(v[e]);
          }
        } else {
          float* c = static_cast<float*>(d.C) + static_cast<int64_t>(sp) * d.split_stride +
                     m * d.ldc + n;
          if (full) {
            float4 o = make_float4(v[0], v[1], v[2], v[3]);
            if constexpr (kEpi == kEpiAccumF32) {
              const float4 old = *reinterpret_cast<const float4*>(c);
              o.x += old.x; o.y += old.y; o.z += old.z; o.w += old.w;
            }
            *reinterpret_cast<float4*>(c) = o;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (n + e < d.N) c[e] = (kEpi == kEpiAccumF32) ? c[e] + v[e] : v[e];
          }
        }
      }
    }
  }
}

}  // namespace mfma

template <bool kAK, bool kBKm, int kEpi>
static hipError_t launch_mfma(const GemmDesc& d, hipStream_t s) {
  using namespace mfma;
  const int64_t tiles_m = (d.M + kBM - 1) / kBM, tiles_n = (d.N + kBN - 1) / kBN;
  const int splits = d.k_splits > 1 ? d.k_splits : 1;
  int64_t k_per = (d.K + splits - 1) / splits;
  k_per = (k_per + kBK - 1) / kBK * kBK;
  const int64_t blocks = tiles_m * tiles_n * splits;
  const size_t lds = 4 * kTileElems * sizeof(uint16_t);  // 128 KiB
  auto kern = k_gemm<kAK, kBKm, kEpi>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  GemmDesc dd = d;
  dd.k_splits = splits;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), lds, s, dd, tiles_m,
                     tiles_n, k_per);
  return hipGetLastError();
}

hipError_t launch_gemm_bf16(const GemmDesc& d, hipStream_t s) {
  if (d.M <= 0 || d.N <= 0) return hipSuccess;
  if (d.a_kmajor && d.b_kmajor && d.epilogue == kEpiLogits) return launch_mfma<true, true, kEpiLogits>(d, s);
  if (d.a_kmajor && !d.b_kmajor && d.epilogue == kEpiStoreF32) return launch_mfma<true, false, kEpiStoreF32>(d, s);
  if (!d.a_kmajor && !d.b_kmajor && d.epilogue == kEpiStoreF32) return launch_mfma<false, false, kEpiStoreF32>(d, s);
  if (!d.a_kmajor && !d.b_kmajor && d.epilogue == kEpiAccumF32) return launch_mfma<false, false, kEpiAccumF32>(d, s);
  return hipErrorInvalidValue;
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
  if (d.a_kmajor && d.b_kmajor && d.epilogue == kEpiLogits) return launch_valu<true, true, kEpiLogits>(d, s);
  if (d.a_kmajor && !d.b_kmajor && d.epilogue == kEpiStoreF32) return launch_valu<true, false, kEpiStoreF32>(d, s);
  if (!d.a_kmajor && !d.b_kmajor && d.epilogue == kEpiStoreF32) return launch_valu<false, false, kEpiStoreF32>(d, s);
  if (!d.a_kmajor && !d.b_kmajor && d.epilogue == kEpiAccumF32) return launch_valu<false, false, kEpiAccumF32>(d, s);
  return hipErrorInvalidValue;
}

}  // namespace lce
