// Dense projection Y = X W^T + bias on gfx950 matrix cores (bf16 operands,
// fp32 accumulation): the value projection V = W_v F + b_v and the output
// projection o = W_o g + b_o ("BEV(三) BEVFormer：Query 参数如何与 Feature 的
// 8 个 Head 交互", sections 3 and 11).
//
// With K = N = 256 the projection moves 512 B in and 512 B (bf16) or 1 KB
// (fp32) out per row for 131 kFLOP, well below the bf16 ridge point, so it is
// bound by HBM, not by the matrix cores.  The design keeps the weights out of
// the memory stream:
//   - a block is 4 waves; wave w owns 64 output columns and holds its 64 x K
//     slice of W in registers as MFMA B operands for the whole (persistent)
//     kernel;
//   - the block walks 32-row tiles of X (tiles split per die, contiguous);
//     each tile is read once from HBM into LDS (fp32 input is rounded to
//     bf16, ties to even, on the way), and every wave reads its A operands
//     from there;
//   - v_mfma_f32_16x16x32_bf16: per tile each wave issues 2 (rows) x 4
//     (columns) x K/32 instructions; accumulators are 2 x 4 x 4 fp32;
//   - epilogue adds the bias and stores fp32, or bf16 rounded to nearest even.
// MFMA operand layout used: lane l supplies row (A) or column (B) l % 16 and
// 8 consecutive k values of a 32-wide k step; result element (i, j) sits in
// lane j + 16*(i/4), register i % 4.
#include "common.hpp"
#include "internal.hpp"

namespace msda {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBM = 32;            // rows per tile
constexpr int kGemmWaves = 4;
constexpr int kColsPerWave = 64;   // 4 MFMA column tiles of 16
constexpr int kBN = kGemmWaves * kColsPerWave;
constexpr int kMaxK = 256;
constexpr int kMaxKSteps = kMaxK / 32;
constexpr int kRowPad = 8;         // bf16 elements of padding per LDS row (spreads banks)

__device__ inline uint32_t bf16_rne_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;  // NaN stays NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ inline uint32_t pack_bf16x2(float lo, float hi) { return bf16_rne_bits(lo) | (bf16_rne_bits(hi) << 16); }

__global__ __launch_bounds__(kGemmWaves* kWave) void gemm_bf16_kernel(GemmArgs a) {
  __shared__ __align__(16) uint16_t xs[kBM][kMaxK + kRowPad];
  const int lane = threadIdx.x % kWave;
  const int wave = uniform(threadIdx.x / kWave);
  const int ksteps = a.K / 32;
  const int col0 = blockIdx.y * kBN + wave * kColsPerWave;
  const int lrow = lane % 16, lk = 8 * (lane / 16);

  // this wave's W slice as B operands, resident for the whole kernel
  bf16x8_t wop[4][kMaxKSteps];
  float bias[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int n = col0 + 16 * nt + lrow;
    bias[nt] = (a.bias && n < a.N) ? a.bias[n] : 0.f;
#pragma unroll
    for (int ks = 0; ks < kMaxKSteps; ++ks) {
      bf16x8_t v = {};
      if (ks < ksteps && n < a.N) v = *reinterpret_cast<const bf16x8_t*>(a.W + (int64_t)n * a.K + 32 * ks + lk);
      wop[nt][ks] = v;
    }
  }

  const int64_t tiles = (a.M + kBM - 1) / kBM;
  const int xcd = blockIdx.x % kXcds, local = blockIdx.x / kXcds, nlocal = gridDim.x / kXcds;
  const int64_t t_end = tiles * (xcd + 1) / kXcds;
  const int chunks = kBM * a.K / 8;  // 8-element chunks per tile
  const int row_chunks = a.K / 8;
  for (int64_t t = tiles * xcd / kXcds + local; t < t_end; t += nlocal) {
    const int64_t m0 = t * kBM;
    for (int e = threadIdx.x; e < chunks; e += kGemmWaves * kWave) {
      const int r = e / row_chunks, kc = (e % row_chunks) * 8;
      const int64_t m = m0 + r;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (m < a.M) {
        if (a.x_f32) {
          const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(a.X) + m * a.K + kc);
          const float4 p = src[0], q = src[1];
          v = make_uint4(pack_bf16x2(p.x, p.y), pack_bf16x2(p.z, p.w), pack_bf16x2(q.x, q.y), pack_bf16x2(q.z, q.w));
        } else {
          v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.X) + m * a.K + kc);
        }
      }
      *reinterpret_cast<uint4*>(&xs[r][kc]) = v;
    }
    __syncthreads();

    f32x4_t acc[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kMaxKSteps; ++ks) {
      if (ks < ksteps) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const bf16x8_t aop = *reinterpret_cast<const bf16x8_t*>(&xs[16 * mt + lrow][32 * ks + lk]);
#pragma unroll
          for (int nt = 0; nt < 4; ++nt)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, wop[nt][ks], acc[mt][nt], 0, 0, 0);
        }
      }
    }
    __syncthreads();  // the next tile overwrites xs

#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int n = col0 + 16 * nt + lrow;
        if (n >= a.N) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t m = m0 + 16 * mt + 4 * (lane / 16) + i;
          if (m >= a.M) continue;
          const float y = acc[mt][nt][i] + bias[nt];
          if (a.y_f32)
            static_cast<float*>(a.Y)[m * a.N + n] = y;
          else
            static_cast<uint16_t*>(a.Y)[m * a.N + n] = (uint16_t)bf16_rne_bits(y);
        }
      }
    }
  }
}

static int gemm_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      cus = n;
    else
      cus = 256;
  }
  return cus;
}

hipError_t launch_gemm_bf16(const GemmArgs& a, hipStream_t stream) {
  const int64_t tiles = (a.M + kBM - 1) / kBM;
  int64_t bx = (int64_t)gemm_cus() * 2;
  if (bx > tiles) bx = tiles;
  bx = (bx + kXcds - 1) / kXcds * kXcds;
  const dim3 grid((unsigned)bx, (unsigned)((a.N + kBN - 1) / kBN));
  gemm_bf16_kernel<<<grid, kGemmWaves * kWave, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace msda
