// Dense projections on gfx950 matrix cores (bf16 operands, fp32 accumulation)
// from "BEV(三) BEVFormer：Query 参数如何与 Feature 的 8 个 Head 交互":
//   - value projection V = W_v F + b_v (section 3);
//   - query projections: offsets W_off q~ + b_off and logits W_att q~ + b_att
//     from q~ = query + position embedding (sections 4.1, 4.2, 18.3), one
//     launch writing both outputs;
//   - output projection o = W_o g + b_o (section 11), optionally followed by
//     the residual and the encoder layer's norm (sections 18.6, 18.7).
//
// With K = 256 a projection moves 512 B in and 512 B (bf16) or 1 KB (fp32)
// out per row and output block for 131 kFLOP, below the bf16 ridge point, so
// it is bound by HBM; the design keeps the X stream flowing and W out of it:
//   - a block is 8 waves over 256 output columns; wave w holds its 32 x K
//     slice of W in registers as MFMA A operands for the whole persistent
//     kernel (grid y covers N beyond 256; the x extent is cut so that all y
//     blocks of one x are resident together on one die and walk the same X
//     tiles, which the die's L2 then serves once);
//   - the block walks 64-row tiles of X (tiles split per die, contiguous),
//     double-buffered in LDS: the loads of tile t+1 are issued before tile t
//     is multiplied and land in the other buffer afterwards (fp32 X, plus the
//     optional float32 addend, is rounded to bf16, ties to even, on the way);
//     16-byte chunks are XOR-swizzled by row so the MFMA operand reads hit 16
//     different banks;
//   - v_mfma_f32_16x16x32_bf16 with W as the A and X as the B operand, so the
//     result tile is transposed: each lane ends with 4 consecutive output
//     columns of one row and stores them with one 16-byte (fp32) or 8-byte
//     (bf16) write, after the bias (and residual / norm) epilogue.
// MFMA operand layout used: lane l supplies row (A) or column (B) l % 16 and
// 8 consecutive k of a 32-wide k step; result element (i, j) sits in lane
// j + 16*(i/4), register i % 4.
#include "common.hpp"
#include "gemm.hpp"

namespace msda {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kGemmWaves = 8;
constexpr int kGemmThreads = kGemmWaves * kWave;
constexpr int kColsPerWave = 32;  // 2 MFMA tiles of 16 columns
constexpr int kBN = kGemmWaves * kColsPerWave;
constexpr int kBM = 64;           // rows per tile: 4 MFMA tiles of 16 rows
constexpr int kMaxK = 256;
constexpr int kMaxKSteps = kMaxK / 32;
constexpr int kChunks = kMaxK / 8;                     // 16-byte chunks per row
constexpr int kLoadsPerThread = kBM * kChunks / kGemmThreads;  // 4
static_assert(kBN == kGemmNormCols, "the norm epilogue needs a whole row in one block");

__device__ inline uint32_t bf16_rne_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;  // NaN stays NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ inline uint32_t pack_bf16x2(float lo, float hi) { return bf16_rne_bits(lo) | (bf16_rne_bits(hi) << 16); }

__device__ inline float4 add4(float4 p, float4 q) { return make_float4(p.x + q.x, p.y + q.y, p.z + q.z, p.w + q.w); }

// swizzled position of 16-byte chunk c of row r inside a tile buffer
__device__ inline int chunk_at(int r, int c) { return r * kChunks + (c ^ (r & 15)); }

template <bool kXAdd>
struct TileLoad {
  uint4 v[kLoadsPerThread];

  // Issue the loads of rows [m0, m0 + kBM) (rows past M read zero).
  __device__ inline void issue(const GemmArgs& a, int64_t m0, int row_chunks) {
#pragma unroll
    for (int i = 0; i < kLoadsPerThread; ++i) {
      const int e = threadIdx.x + i * kGemmThreads;
      const int r = e / kChunks, c = e % kChunks;
      const int64_t m = m0 + r;
      v[i] = make_uint4(0u, 0u, 0u, 0u);
      if (c < row_chunks && m < a.M) {
        if (a.x_f32) {
          const int64_t at = m * a.K + 8 * c;
          const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(a.X) + at);
          float4 p = src[0], q = src[1];
          if constexpr (kXAdd) {
            const float4* add = reinterpret_cast<const float4*>(a.X_add + at);
            p = add4(p, add[0]);
            q = add4(q, add[1]);
          }
          v[i] = make_uint4(pack_bf16x2(p.x, p.y), pack_bf16x2(p.z, p.w), pack_bf16x2(q.x, q.y),
                            pack_bf16x2(q.z, q.w));
        } else {
          v[i] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.X) + m * a.K + 8 * c);
        }
      }
    }
  }

  __device__ inline void store(uint4* buf) const {
#pragma unroll
    for (int i = 0; i < kLoadsPerThread; ++i) {
      const int e = threadIdx.x + i * kGemmThreads;
      buf[chunk_at(e / kChunks, e % kChunks)] = v[i];
    }
  }
};

__device__ inline float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }
// four floats with only 4-byte alignment (per-column parameters, read once)
__device__ inline float4 load4s(const float* p) { return make_float4(p[0], p[1], p[2], p[3]); }

// kXAdd: X is float32 with a float32 addend.  kNorm: one output of N == 256
// columns followed by the layer norm of each row.
template <bool kXAdd, bool kNorm>
__global__ __launch_bounds__(kGemmThreads) void gemm_bf16_kernel(GemmArgs a) {
  __shared__ uint4 xs[2][kBM * kChunks];  // two 64 x 256 bf16 tiles, 64 KB
  const int lane = threadIdx.x % kWave;
  const int wave = uniform((int)(threadIdx.x / kWave));
  const int ksteps = a.K / 32;
  const int row_chunks = a.K / 8;
  const int l16 = lane % 16, lg = lane / 16;

  // the output part this wave's 32 columns fall in (N1 % 32 == 0)
  const int col = blockIdx.y * kBN + wave * kColsPerWave;
  const bool first = col < a.N1;
  const int c0 = first ? col : col - a.N1;  // first column inside the part
  const int Np = first ? a.N1 : a.N - a.N1;  // columns of the part
  const uint16_t* W = first ? a.W1 : a.W2;
  const float* bias_p = first ? a.bias1 : a.bias2;
  void* Y = first ? a.Y1 : a.Y2;

  // this wave's W slice as A operands, resident for the whole kernel
  bf16x8_t wop[2][kMaxKSteps];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int n = c0 + 16 * nt + l16;
#pragma unroll
    for (int ks = 0; ks < kMaxKSteps; ++ks) {
      bf16x8_t v = {};
      if (ks < ksteps && n < Np) v = *reinterpret_cast<const bf16x8_t*>(W + (int64_t)n * a.K + 32 * ks + 8 * lg);
      wop[nt][ks] = v;
    }
  }
  // bias (and norm scale and shift) of the 4 output columns this lane stores per column tile
  float4 bias[2], gam[2], bet[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int n = c0 + 16 * nt + 4 * lg;
    const bool in = n < Np;
    bias[nt] = bias_p && in ? load4s(bias_p + n) : make_float4(0.f, 0.f, 0.f, 0.f);
    if constexpr (kNorm) {
      gam[nt] = load4s(a.gamma + n);
      bet[nt] = a.beta ? load4s(a.beta + n) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }

  const int64_t tiles = (a.M + kBM - 1) / kBM;
  const int xcd = blockIdx.x % kXcds, local = blockIdx.x / kXcds, nlocal = gridDim.x / kXcds;
  const int64_t t_begin = tiles * xcd / kXcds + local, t_end = tiles * (xcd + 1) / kXcds;
  if (t_begin >= t_end) return;  // uniform over the block

  TileLoad<kXAdd> next;
  next.issue(a, t_begin * kBM, row_chunks);
  next.store(xs[0]);
  __syncthreads();
  int buf = 0;
  for (int64_t t = t_begin; t < t_end; t += nlocal) {
    const int64_t t_next = t + nlocal;
    if (t_next < t_end) next.issue(a, t_next * kBM, row_chunks);  // in flight during the MFMAs

    f32x4_t acc[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const uint4* cur = xs[buf];
#pragma unroll
    for (int ks = 0; ks < kMaxKSteps; ++ks) {
      if (ks < ksteps) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const uint4 raw = cur[chunk_at(16 * mt + l16, 4 * ks + lg)];
          const bf16x8_t xop = __builtin_bit_cast(bf16x8_t, raw);
#pragma unroll
          for (int nt = 0; nt < 2; ++nt)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wop[nt][ks], xop, acc[mt][nt], 0, 0, 0);
        }
      }
    }

    // acc[mt][nt][i] = Y[m0 + 16 mt + l16][c0 + 16 nt + 4 lg + i]
    const int64_t m0 = t * kBM;
    float4 y[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int64_t m = m0 + 16 * mt + l16;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int n = c0 + 16 * nt + 4 * lg;
        y[mt][nt] = make_float4(acc[mt][nt][0] + bias[nt].x, acc[mt][nt][1] + bias[nt].y,
                                acc[mt][nt][2] + bias[nt].z, acc[mt][nt][3] + bias[nt].w);
        if (a.residual && m < a.M && n < Np) y[mt][nt] = add4(y[mt][nt], load4(a.residual + m * Np + n));
      }
    }
    if constexpr (kNorm) {
      // row statistics over the 256 columns: 8 values per lane, the 4 lanes
      // of one row in a wave (xor 16, 32), then the 8 waves through LDS
      __shared__ float red[2][kGemmWaves][kBM];
      constexpr float kInvN = 1.0f / kGemmNormCols;
      // pairwise over the 8 waves (a constant row then sums exactly)
      auto wave_sum = [&](int k, int row) {
        const float* r = &red[k][0][row];
        return ((r[0] + r[kBM]) + (r[2 * kBM] + r[3 * kBM])) + ((r[4 * kBM] + r[5 * kBM]) + (r[6 * kBM] + r[7 * kBM]));
      };
      static_assert(kGemmWaves == 8, "wave_sum adds 8 partial sums");
      float mean[4], rstd[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        float s = 0.f;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) s += (y[mt][nt].x + y[mt][nt].y) + (y[mt][nt].z + y[mt][nt].w);
        s += __shfl_xor(s, 16);
        s += __shfl_xor(s, 32);
        if (lg == 0) red[0][wave][16 * mt + l16] = s;
      }
      __syncthreads();
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        mean[mt] = wave_sum(0, 16 * mt + l16) * kInvN;
        float q = 0.f;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const float4 d = make_float4(y[mt][nt].x - mean[mt], y[mt][nt].y - mean[mt], y[mt][nt].z - mean[mt],
                                       y[mt][nt].w - mean[mt]);
          q += (d.x * d.x + d.y * d.y) + (d.z * d.z + d.w * d.w);
        }
        q += __shfl_xor(q, 16);
        q += __shfl_xor(q, 32);
        if (lg == 0) red[1][wave][16 * mt + l16] = q;
      }
      __syncthreads();
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        rstd[mt] = 1.0f / sqrtf(wave_sum(1, 16 * mt + l16) * kInvN + a.eps);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const float4 g = gam[nt], b = bet[nt];
          float4& v = y[mt][nt];
          v = make_float4((v.x - mean[mt]) * rstd[mt] * g.x + b.x, (v.y - mean[mt]) * rstd[mt] * g.y + b.y,
                          (v.z - mean[mt]) * rstd[mt] * g.z + b.z, (v.w - mean[mt]) * rstd[mt] * g.w + b.w);
        }
      }
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int64_t m = m0 + 16 * mt + l16;
      if (m >= a.M) continue;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int n = c0 + 16 * nt + 4 * lg;
        if (n >= Np) continue;
        if (a.y_f32) {
          *reinterpret_cast<float4*>(static_cast<float*>(Y) + m * Np + n) = y[mt][nt];
        } else {
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(Y) + m * Np + n) =
              make_uint2(pack_bf16x2(y[mt][nt].x, y[mt][nt].y), pack_bf16x2(y[mt][nt].z, y[mt][nt].w));
        }
      }
    }

    if (t_next < t_end) next.store(xs[buf ^ 1]);
    __syncthreads();  // the next tile is in place and nobody reads this one any more
    buf ^= 1;
  }
}

static int gemm_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      cus = n;
    else
      cus = 256;
  }
  return cus;
}

hipError_t launch_gemm_bf16(const GemmArgs& a, hipStream_t stream) {
  const int64_t tiles = (a.M + kBM - 1) / kBM;
  const int64_t gy = (a.N + kBN - 1) / kBN;
  // one 8-wave block per CU (register-bound); with several column blocks the
  // x extent is cut so that all of them fit on the chip at once
  int64_t bx = gemm_cus() / gy / kXcds * kXcds;
  if (bx < kXcds) bx = kXcds;
  const int64_t tiles_up = (tiles + kXcds - 1) / kXcds * kXcds;
  if (bx > tiles_up) bx = tiles_up;
  const dim3 grid((unsigned)bx, (unsigned)gy);
  // the norm epilogue is used for the output projection only, which has no addend
  const bool add = a.X_add != nullptr, norm = a.gamma != nullptr;
  if (norm)
    gemm_bf16_kernel<false, true><<<grid, kGemmThreads, 0, stream>>>(a);
  else if (add)
    gemm_bf16_kernel<true, false><<<grid, kGemmThreads, 0, stream>>>(a);
  else
    gemm_bf16_kernel<false, false><<<grid, kGemmThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace msda
