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
//   - the block walks tiles of 64 rows of X (32 where the registers would not
//     hold more; tiles split per die, contiguous), double-buffered in LDS,
//     with two tiles in flight per thread: while tile t is multiplied, tiles
//     t+1 and t+2 are loading into registers, and tile t+1 lands in the other
//     buffer afterwards; float32 X (plus the optional float32 addend) stays
//     raw in registers while in flight and is rounded to bf16, ties to even,
//     by v_cvt_pk_bf16_f32 on its way into LDS.  16-byte chunks are
//     XOR-swizzled by row so the MFMA operand reads hit 16 different banks;
//   - every tile access (X, addend, residual, output) goes through a buffer
//     descriptor spanning the tile's rows: rows past M and absent chunks read
//     zero or drop their store with no branch;
//   - v_mfma_f32_16x16x32_bf16 with W as the A and X as the B operand, so the
//     result tile is transposed: each lane ends with 4 consecutive output
//     columns of one row; after the bias (and residual / norm) epilogue the
//     tile goes through LDS and out as whole rows, consecutive lanes writing
//     consecutive 16-byte chunks (writing straight from the MFMA layout, 8
//     or 16 bytes per lane in 32- or 64-byte row pieces, made the stores the
//     bottleneck).
// MFMA operand layout used: lane l supplies row (A) or column (B) l % 16 and
// 8 consecutive k of a 32-wide k step; result element (i, j) sits in lane
// j + 16*(i/4), register i % 4.
#include "common.hpp"
#include "gemm.hpp"

namespace msda {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kGemmWaves = 8;
constexpr int kGemmThreads = kGemmWaves * kWave;
constexpr int kColsPerWave = 32;  // 2 MFMA tiles of 16 columns
constexpr int kBN = kGemmWaves * kColsPerWave;
constexpr int kMaxK = 256;
constexpr int kMaxKSteps = kMaxK / 32;
constexpr int kChunks = kMaxK / 8;  // 16-byte bf16 chunks per row
constexpr uint32_t kAbsent = 0x80000000u;  // offset past every tile descriptor: reads 0, drops stores
static_assert(kBN == kGemmNormCols, "the norm epilogue needs a whole row in one block");

// rows per tile: 64, or 32 where the tiles in flight and the epilogue's
// operands would not fit the registers otherwise (a float32 addend, a
// residual, the norm)
template <bool kXAdd, bool kRes, bool kNorm>
constexpr int rows_per_tile() { return kXAdd || kRes || kNorm ? 32 : 64; }

// two floats to two bf16 (round to nearest even) in one 32-bit word, low first
__device__ inline uint32_t cvt2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

__device__ inline float4 add4(float4 p, float4 q) { return make_float4(p.x + q.x, p.y + q.y, p.z + q.z, p.w + q.w); }
__device__ inline float4 as_f4(u32x4_t v) { return __builtin_bit_cast(float4, v); }

// swizzled position of 16-byte chunk c of row r inside a tile buffer
__device__ inline int chunk_at(int r, int c) { return r * kChunks + (c ^ (r & 15)); }

// Descriptor over rows [m0, min(m0 + rows, M)) of a row-major matrix with
// `row_bytes` bytes per row: rows past M read zero (m0 >= M: an empty range).
__device__ inline __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, int64_t m0, int64_t M, int rows,
                                                   int64_t row_bytes) {
  int64_t n = M - m0 < rows ? M - m0 : rows;
  if (n < 0) n = 0;
  return make_rsrc(static_cast<const char*>(base) + m0 * row_bytes, (uint32_t)(n * row_bytes));
}

// One thread's share of a tile of X: kLoads 16-byte bf16 chunks, loaded raw
// (float32 chunks are two 16-byte halves, plus the addend's) and packed to
// bf16 when stored into LDS.
template <bool kXF32, bool kXAdd, int kRows>
struct TileLoad {
  static constexpr int kBM = kRows;
  static constexpr int kLoads = kBM * kChunks / kGemmThreads;
  static constexpr int kHalves = kXF32 ? 2 : 1;
  static constexpr int kSrc = kXAdd ? 2 : 1;
  static constexpr int kElem = kXF32 ? 4 : 2;
  u32x4_t raw[kSrc][kLoads][kHalves];
  uint32_t off[kLoads];  // byte offset of each chunk inside the tile, or kAbsent

  __device__ inline void init(int K) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int e = threadIdx.x + i * kGemmThreads;
      const int r = e / kChunks, c = e % kChunks;
      off[i] = 8 * c < K ? (uint32_t)((r * K + 8 * c) * kElem) : kAbsent;
    }
  }

  __device__ inline void issue(const GemmArgs& a, int64_t m0) {
    const int64_t row_bytes = (int64_t)a.K * kElem;
#pragma unroll
    for (int s = 0; s < kSrc; ++s) {
      const auto rs = tile_rsrc(s == 0 ? a.X : a.X_add, m0, a.M, kBM, row_bytes);
#pragma unroll
      for (int i = 0; i < kLoads; ++i)
#pragma unroll
        for (int h = 0; h < kHalves; ++h) raw[s][i][h] = __builtin_amdgcn_raw_buffer_load_b128(rs, off[i] + 16 * h, 0, 0);
    }
  }

  __device__ inline void store(uint4* buf) const {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int e = threadIdx.x + i * kGemmThreads;
      uint4 v;
      if constexpr (kXF32) {
        float4 p = as_f4(raw[0][i][0]), q = as_f4(raw[0][i][1]);
        if constexpr (kXAdd) {
          p = add4(p, as_f4(raw[1][i][0]));
          q = add4(q, as_f4(raw[1][i][1]));
        }
        v = make_uint4(cvt2(p.x, p.y), cvt2(p.z, p.w), cvt2(q.x, q.y), cvt2(q.z, q.w));
      } else {
        v = __builtin_bit_cast(uint4, raw[0][i][0]);
      }
      buf[chunk_at(e / kChunks, e % kChunks)] = v;
    }
  }
};

// four floats with only 4-byte alignment (per-column parameters, read once)
__device__ inline float4 load4s(const float* p) { return make_float4(p[0], p[1], p[2], p[3]); }

// kXF32: X is float32 (rounded to bf16 on the way into LDS).  kXAdd: plus a
// float32 addend.  kRes: a float32 residual is added to the single output.
// kNorm: one output of N == 256 columns followed by the layer norm of each
// row.  kYF32: float32 output (else bf16).  Fixed at compile time so that the
// waits the compiler places never cover loads that are meant to stay in
// flight.
template <bool kXF32, bool kXAdd, bool kRes, bool kNorm, bool kYF32>
__global__ __launch_bounds__(kGemmThreads) void gemm_bf16_kernel(GemmArgs a) {
  using Tile = TileLoad<kXF32, kXAdd, rows_per_tile<kXAdd, kRes, kNorm>()>;
  constexpr int kBM = Tile::kBM;
  constexpr int kMT = kBM / 16;  // MFMA row tiles per tile
  __shared__ uint4 xs[2][kBM * kChunks];  // two bf16 tiles of kBM x 256
  __shared__ float red[2][kGemmWaves][kNorm ? kBM : 1];  // norm: per-wave row sums
  const int lane = threadIdx.x % kWave;
  const int wave = uniform((int)(threadIdx.x / kWave));
  const int ksteps = a.K / 32;
  const int l16 = lane % 16, lg = lane / 16;

  // the output part this wave's 32 columns fall in (N1 % 32 == 0)
  const int col = blockIdx.y * kBN + wave * kColsPerWave;
  const bool first = col < a.N1;
  const int c0 = first ? col : col - a.N1;  // first column inside the part
  const int Np = first ? a.N1 : a.N - a.N1;  // columns of the part
  const uint16_t* W = first ? a.W1 : a.W2;
  const float* bias_p = first ? a.bias1 : a.bias2;
  constexpr int ysz = kYF32 ? 4 : 2;

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
  // per column tile: bias (and norm scale and shift) of this lane's 4 output
  // columns, and their element offset inside a row of the part (or absent)
  float4 bias[2], gam[2], bet[2];
  int ncol[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int n = c0 + 16 * nt + 4 * lg;
    const bool in = n < Np;
    ncol[nt] = in ? n : -1;
    bias[nt] = bias_p && in ? load4s(bias_p + n) : make_float4(0.f, 0.f, 0.f, 0.f);
    if constexpr (kNorm) {
      gam[nt] = load4s(a.gamma + n);
      bet[nt] = a.beta ? load4s(a.beta + n) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  // byte offsets of this lane's outputs inside a tile of the part (element
  // size esz), kAbsent for columns past the part
  auto out_off = [&](int mt, int nt, int esz) -> uint32_t {
    return ncol[nt] < 0 ? kAbsent : (uint32_t)(((16 * mt + l16) * Np + ncol[nt]) * esz);
  };

  const int64_t tiles = (a.M + kBM - 1) / kBM;
  const int xcd = blockIdx.x % kXcds, local = blockIdx.x / kXcds, nlocal = gridDim.x / kXcds;
  const int64_t t_begin = tiles * xcd / kXcds + local, t_end = tiles * (xcd + 1) / kXcds;
  if (t_begin >= t_end) return;  // uniform over the block

  // Output staging: kBM rows of this block's 256 columns, rows padded by 16
  // bytes so that the 16 rows a store instruction touches spread over the
  // banks.  Chunk e of the tile (16 bytes) is row e / kRowChunks, column
  // chunk e % kRowChunks; its columns belong to one output part (N1 % 32 == 0).
  constexpr int kRowChunks = kBN * ysz / 16;
  constexpr int kYPitch = kBN * ysz + 16;
  constexpr int kOutChunks = kBM * kRowChunks / kGemmThreads;
  constexpr int kColsPerChunk = 16 / ysz;
  __shared__ __align__(16) char ys[kBM * kYPitch];
  // Head-pair layout (msda_value_proj_pairs_bf16): row m = pixel pix of
  // image m / Nv, columns h*32 .. h*32+31 = head h.  Its 16-byte chunk o of
  // head h goes to the left half of line (h, pix) and to the right half of
  // line (h, pix - 1); the right half of the image's last line is zeroed.
  // Lanes take consecutive rows of one head, so that a wave's two stores
  // cover whole consecutive lines.
  auto store_pairs = [&](int64_t m0) {
    const int64_t Nv = a.pairs_Nv;
    const int64_t image_bytes = Nv * (a.N / 32) * 128;
    char* Y = static_cast<char*>(a.Y1);
#pragma unroll
    for (int i = 0; i < kOutChunks; ++i) {
      const int e = threadIdx.x + i * kGemmThreads;
      const int o = e % 4, r = (e / 4) % kBM, hb = e / (4 * kBM);  // head within the block's 8
      const int64_t m = m0 + r;
      const int h = blockIdx.y * (kBN / 32) + hb;
      if (m >= a.M || h * 32 >= a.N) continue;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(ys + r * kYPitch + (hb * 4 + o) * 16);
      const uint32_t img = (uint32_t)m / (uint32_t)Nv;  // m < 2^31
      const int64_t pix = m - (int64_t)img * Nv;
      char* line = Y + img * image_bytes + ((int64_t)h * Nv + pix) * 128 + o * 16;
      *reinterpret_cast<u32x4_t*>(line) = v;
      if (pix > 0) *reinterpret_cast<u32x4_t*>(line - 64) = v;
      if (pix == Nv - 1) *reinterpret_cast<u32x4_t*>(line + 64) = u32x4_t{0u, 0u, 0u, 0u};
    }
  };
  const bool straddles = blockIdx.y * kBN < a.N1 && (blockIdx.y + 1) * kBN > a.N1;  // uniform
  const bool all2 = blockIdx.y * kBN >= a.N1;  // uniform
  auto store_tile = [&](int64_t m0) {
    if constexpr (!kYF32) {
      if (a.pairs_Nv > 0) {  // uniform: the head-pair layout (single output, bf16)
        store_pairs(m0);
        return;
      }
    }
    const auto r1 = tile_rsrc(a.Y1, m0, a.M, kBM, (int64_t)a.N1 * ysz);
    const auto r2 = tile_rsrc(a.Y2, m0, a.M, kBM, (int64_t)(a.N - a.N1) * ysz);
#pragma unroll
    for (int i = 0; i < kOutChunks; ++i) {
      const int e = threadIdx.x + i * kGemmThreads;
      const int r = e / kRowChunks, cc = e % kRowChunks;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(ys + r * kYPitch + cc * 16);
      const int gc = blockIdx.y * kBN + cc * kColsPerChunk;  // column over both parts
      const bool p2 = gc >= a.N1;
      const uint32_t off = gc < a.N ? (uint32_t)((r * (p2 ? a.N - a.N1 : a.N1) + (p2 ? gc - a.N1 : gc)) * ysz)
                                    : kAbsent;  // past N: dropped
      if (straddles) {  // the block's columns cover both parts: one store each, one of them dropped
        __builtin_amdgcn_raw_buffer_store_b128(v, r1, p2 ? kAbsent : off, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(v, r2, p2 ? off : kAbsent, 0, 0);
      } else {
        __builtin_amdgcn_raw_buffer_store_b128(v, all2 ? r2 : r1, off, 0, 0);
      }
    }
  };

  int buf = 0;
  // Two tiles in flight per thread: while tile t is multiplied, tile t + 1
  // (issued one step earlier) and tile t + 2 (issued now) are loading; the
  // loop is unrolled by two so each load set keeps its own registers.
  auto step = [&](int64_t t, Tile& fill, const Tile& land) {
    const int64_t m0 = t * kBM;
    const int64_t t_fill = t + 2 * nlocal;
    // residual of this tile first, then the tile after next: waiting for
    // the residual leaves both tiles in flight
    float4 res[kMT][2];
    if constexpr (kRes) {
      const auto rr = tile_rsrc(a.residual, m0, a.M, kBM, (int64_t)Np * 4);
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) res[mt][nt] = as_f4(__builtin_amdgcn_raw_buffer_load_b128(rr, out_off(mt, nt, 4), 0, 0));
    }
    // past the last tile an empty range (no memory request), so that the
    // loop body has no branch around loads
    fill.issue(a, t_fill < t_end ? t_fill * kBM : a.M);

    f32x4_t acc[kMT][2];
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const uint4* cur = xs[buf];
#pragma unroll
    for (int ks = 0; ks < kMaxKSteps; ++ks) {
      if (ks < ksteps) {
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
          const uint4 raw = cur[chunk_at(16 * mt + l16, 4 * ks + lg)];
          const bf16x8_t xop = __builtin_bit_cast(bf16x8_t, raw);
#pragma unroll
          for (int nt = 0; nt < 2; ++nt)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wop[nt][ks], xop, acc[mt][nt], 0, 0, 0);
        }
      }
    }

    // acc[mt][nt][i] = Y[m0 + 16 mt + l16][c0 + 16 nt + 4 lg + i]
    float4 y[kMT][2];
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        y[mt][nt] = make_float4(acc[mt][nt][0] + bias[nt].x, acc[mt][nt][1] + bias[nt].y,
                                acc[mt][nt][2] + bias[nt].z, acc[mt][nt][3] + bias[nt].w);
        if constexpr (kRes) y[mt][nt] = add4(y[mt][nt], res[mt][nt]);
      }
    if constexpr (kNorm) {
      // row statistics over the 256 columns: 8 values per lane, the 4 lanes
      // of one row in a wave (xor 16, 32), then the 8 waves through LDS
      constexpr float kInvN = 1.0f / kGemmNormCols;
      // pairwise over the 8 waves (a constant row then sums exactly)
      auto wave_sum = [&](int k, int row) {
        const float* r = &red[k][0][row];
        return ((r[0] + r[kBM]) + (r[2 * kBM] + r[3 * kBM])) + ((r[4 * kBM] + r[5 * kBM]) + (r[6 * kBM] + r[7 * kBM]));
      };
      static_assert(kGemmWaves == 8, "wave_sum adds 8 partial sums");
      float mean[kMT];
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) {
        float s = 0.f;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) s += (y[mt][nt].x + y[mt][nt].y) + (y[mt][nt].z + y[mt][nt].w);
        s += __shfl_xor(s, 16);
        s += __shfl_xor(s, 32);
        if (lg == 0) red[0][wave][16 * mt + l16] = s;
      }
      __syncthreads();
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) {
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
      for (int mt = 0; mt < kMT; ++mt) {
        const float rstd = 1.0f / sqrtf(wave_sum(1, 16 * mt + l16) * kInvN + a.eps);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const float4 g = gam[nt], b = bet[nt];
          float4& v = y[mt][nt];
          v = make_float4((v.x - mean[mt]) * rstd * g.x + b.x, (v.y - mean[mt]) * rstd * g.y + b.y,
                          (v.z - mean[mt]) * rstd * g.z + b.z, (v.w - mean[mt]) * rstd * g.w + b.w);
        }
      }
    }
    // the tile's outputs go through LDS so that the stores are whole rows:
    // consecutive lanes write consecutive 16-byte chunks
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const float4 v = y[mt][nt];
        char* at = ys + (16 * mt + l16) * kYPitch + (wave * kColsPerWave + 16 * nt + 4 * lg) * ysz;
        if constexpr (kYF32)
          *reinterpret_cast<float4*>(at) = v;
        else
          *reinterpret_cast<uint2*>(at) = make_uint2(cvt2(v.x, v.y), cvt2(v.z, v.w));
      }
    __syncthreads();
    store_tile(m0);
    land.store(xs[buf ^ 1]);  // tile t + 1; zeros past the last tile, never read
    __syncthreads();  // it is in place and nobody reads tile t any more
    buf ^= 1;
  };
  Tile A, B;
  A.init(a.K);
  B.init(a.K);
  A.issue(a, t_begin * kBM);
  A.store(xs[0]);
  __syncthreads();
  B.issue(a, t_begin + nlocal < t_end ? (t_begin + nlocal) * kBM : a.M);
  for (int64_t t = t_begin; t < t_end; t += 2 * nlocal) {
    step(t, A, B);
    if (t + nlocal >= t_end) break;
    step(t + nlocal, B, A);
  }
}


template <bool kXF32, bool kXAdd, bool kRes, bool kNorm, bool kYF32>
static hipError_t launch(const GemmArgs& a, hipStream_t stream) {
  constexpr int kBM = rows_per_tile<kXAdd, kRes, kNorm>();
  const int64_t tiles = (a.M + kBM - 1) / kBM;
  const int64_t gy = (a.N + kBN - 1) / kBN;
  // one 8-wave block per CU (register-bound); with several column blocks the
  // x extent is cut so that all of them fit on the chip at once
  int64_t bx = device_cu_count() / gy / kXcds * kXcds;
  if (bx < kXcds) bx = kXcds;
  const int64_t tiles_up = (tiles + kXcds - 1) / kXcds * kXcds;
  if (bx > tiles_up) bx = tiles_up;
  gemm_bf16_kernel<kXF32, kXAdd, kRes, kNorm, kYF32><<<dim3((unsigned)bx, (unsigned)gy), kGemmThreads, 0, stream>>>(a);
  return hipGetLastError();
}

// The variants the entry points use: the addend comes with float32 X and
// float32 output only (query projections); residual and norm come with
// float32 output only (output projection).
template <bool kXF32>
static hipError_t launch_output_side(const GemmArgs& a, hipStream_t stream) {
  if (a.gamma)
    return a.residual ? launch<kXF32, false, true, true, true>(a, stream)
                      : launch<kXF32, false, false, true, true>(a, stream);
  if (a.residual) return launch<kXF32, false, true, false, true>(a, stream);
  return a.y_f32 ? launch<kXF32, false, false, false, true>(a, stream)
                 : launch<kXF32, false, false, false, false>(a, stream);
}

hipError_t launch_gemm_bf16(const GemmArgs& a, hipStream_t stream) {
  if (a.X_add) return launch<true, true, false, false, true>(a, stream);
  return a.x_f32 ? launch_output_side<true>(a, stream) : launch_output_side<false>(a, stream);
}

}  // namespace msda
