// Split-K decode attention on the matrix cores (bf16 KV, D in {64, 128}).
//
// Same result as the VALU kernel -- softmax(q K^T * scale) V per (b, h),
// "Transformer推理核心：KV Cache、GQA与RoPE原理与工程实践" §2.1/§4.2 -- with the
// two products of each 32-token tile done by v_mfma_f32_16x16x32_bf16.  The
// query heads of one KV head are the 16 columns of the MFMA (two passes of
// 16 for n_rep up to 32), so one K/V tile read from HBM feeds all n_rep heads
// (the GQA sharing of §2.2 of the same page, without materialising the
// broadcast).
//
// Per wave and 32-token tile:
//   scores  S[t][h] = sum_d K[t][d] q[h][d]: A = K rows straight from HBM in
//           the A-operand layout (lane = token row, 8 dims per lane), B = q.
//           q is fp32; it enters the bf16 product as q_hi + q_lo, two bf16
//           numbers whose sum is q to ~2^-17, as two MFMAs into one
//           accumulator, so scores keep near-fp32 accuracy while K is exact.
//   softmax the score output puts head h in lane h % 16 with tokens
//           16*tb + 4*(lane/16) + j; running max and sum per head live in
//           that lane, the tile max crosses the 4 lane groups with two
//           shuffles, and the accumulators are rescaled only when some
//           running max actually moved.
//   P V     computed transposed, O^T[d][h] += sum_t V[t][d] P[h][t]: the B
//           operand P^T needs exactly the probabilities the lane holds (the
//           token order inside the contraction is free and chosen to match
//           the score layout), and each head's accumulators stay in its
//           lanes, so the rescale moves no data.  P is split hi + lo like q.
//           V^T is the A operand.  V rows travel HBM -> LDS directly
//           (global_load_lds, 16 bytes per lane, no registers): each
//           instruction lands 64 lanes x 16 bytes contiguously, rows in
//           order, and consecutive instructions are 32 bytes apart, so the
//           four lane groups' 2-byte column reads fall in disjoint banks.
//           Rows past the end of the sequence are zeroed in LDS after the
//           copy (padding may hold NaN and 0 * NaN is NaN).
//
// Software pipeline: while tile i is computed, tile i+1 is in flight -- its V
// rows into the second of two LDS buffers from the start of tile i, its K
// rows into the K registers as soon as tile i's score MFMAs have read them --
// so a wave keeps up to 16 KB of loads outstanding while it works.
// Vector-memory loads complete in issue order, so "at most N outstanding"
// (s_waitcnt vmcnt(N), N = the loads of one tile) says tile i has landed.
// Paged block ids are staged in LDS once per workgroup, so no table load
// sits between two tiles' loads.  Waves of a workgroup take interleaved
// tiles of the split and merge their (m, l, O) through LDS at the end.
#include "kvd_internal.h"

namespace kvd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void* lds_ptr;

constexpr float kNegInf = -__builtin_inff();
constexpr int kMaxChunkBlocks = kMfmaMaxChunk / 16;

// bf16 bits of a finite float, nearest-even.
__device__ __forceinline__ unsigned short bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<unsigned short>(u >> 16);
}
__device__ __forceinline__ float bf16_value(unsigned short h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
// x ~= hi + lo with both bf16 (the residual x - hi is exact in fp32)
__device__ __forceinline__ void split_bf16(float x, unsigned short& hi, unsigned short& lo) {
  hi = bf16_bits(x);
  lo = bf16_bits(x - bf16_value(hi));
}

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Completes this wave's outstanding LDS accesses and keeps the compiler
// from moving memory accesses across: the wave-private staging tiles are
// written by some lanes and read by others.
__device__ __forceinline__ void lds_fence() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}
// At most N of this wave's vector-memory loads (HBM -> LDS copies included)
// are still outstanding; loads complete in issue order.
template <int N>
__device__ __forceinline__ void vmem_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
  __builtin_amdgcn_wave_barrier();
}

template <int D>
struct Geo {
  static constexpr int KB = D / 32;          // 32-dim blocks of the score contraction
  static constexpr int CB = D / 16;          // 16-dim blocks of the output
  static constexpr int TT = kMfmaTileTokens; // 32 tokens per wave tile
  static constexpr int LPR = D / 8;          // lanes per V row (16 bytes each)
  static constexpr int RPI = 64 / LPR;       // V rows per load instruction
  static constexpr int NVL = TT / RPI;       // V load instructions per tile
  static constexpr int NLOADS = 2 * KB + NVL;  // vector-memory loads per tile
  // every V copy instruction writes 1 KiB; instruction blocks are padded by
  // 32 bytes so the transposed column reads of the four lane groups fall in
  // different banks
  static constexpr int BLOCK = 1024 + 32;
  static constexpr int kTileBytes = NVL * BLOCK;
  // byte offset of (token row r, byte c within the row) in a staged tile
  __device__ __forceinline__ static int at(int r, int c) {
    return (r / RPI) * BLOCK + (r % RPI) * (2 * D) + c;
  }
};

template <int D, int NB, bool PAGED>
__global__ __launch_bounds__(256) void decode_mfma_kernel(DecodeParams p) {
  using G = Geo<D>;
  constexpr int KB = G::KB, CB = G::CB, TT = G::TT, LPR = G::LPR, RPI = G::RPI, NVL = G::NVL;
  constexpr int kWaves = kMfmaWaves;
  constexpr int kStageBytes = kWaves * 2 * G::kTileBytes;         // two V buffers per wave
  constexpr int kMergeBytes = (kWaves * 16 * D + 2 * kWaves * 16) * 4;
  constexpr int kSmem = kStageBytes > kMergeBytes ? kStageBytes : kMergeBytes;
  static_assert(TT == 32 && NB >= 1 && NB <= 2, "tile shape");
  __shared__ __align__(16) char smem[kSmem];
  __shared__ int sm_blk[PAGED ? kMaxChunkBlocks : 1];
  // q_hi / q_lo as B operands: [nb][kb][hi, lo][lane] x 16 bytes
  __shared__ __align__(16) uint4 sm_q[NB * KB * 2 * 64];

  // grid order (chosen by the planner): which of (sequence, KV head, split)
  // varies fastest in dispatch order decides how the workgroups reading the
  // same DRAM rows (the heads of one token range) and the longest chunks are
  // spread in time and across the XCDs
  int b, g, split;
  if (p.grid_order == 0) { split = blockIdx.x; g = blockIdx.y; b = blockIdx.z; }
  else if (p.grid_order == 1) { g = blockIdx.x; b = blockIdx.y; split = blockIdx.z; }
  else { g = blockIdx.x; split = blockIdx.y; b = blockIdx.z; }
  const int R = p.R;
  const int hbase = g * R;            // first query head of this KV head
  int L = __builtin_amdgcn_readfirstlane(p.seq_lens[b]);
  L = L < 0 ? 0 : (L > p.max_len_host ? p.max_len_host : L);
  const int t0 = split * p.chunk;
  if (t0 >= L) {
    if (p.direct && split == 0) {     // empty sequence: out = 0, lse = -inf
      for (int idx = threadIdx.x; idx < R * D; idx += 256) {
        const int r = idx / D, d = idx - r * D;
        p.out[(static_cast<int64_t>(b) * p.H + hbase + r) * D + d] = 0.f;
        if (d == 0 && p.lse) p.lse[static_cast<int64_t>(b) * p.H + hbase + r] = kNegInf;
      }
    }
    return;
  }
  const int t1 = min(t0 + p.chunk, L);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, grp = lane >> 4;
  const char* kbase = static_cast<const char*>(p.k);
  const char* vbase = static_cast<const char*>(p.v);

  if (PAGED) {
    // this split's block ids (an id outside the pool is replaced by -1)
    const int nblk = (t1 - t0 + 15) >> 4;
    for (int i = threadIdx.x; i < nblk; i += 256) {
      const int blk = p.table[static_cast<int64_t>(b) * p.max_blocks_per_seq + (t0 >> 4) + i];
      sm_blk[i] = (blk >= 0 && blk < p.num_blocks) ? blk : -1;
    }
    __syncthreads();
  }
  // row (in units of D elements) of token t of this sequence and KV head; a
  // token in a bad block reads block 0 and is masked out
  auto row_of = [&](int t) -> int64_t {
    if (!PAGED) return (static_cast<int64_t>(b) * p.max_seq_len + t) * p.G + g;
    int blk = sm_blk[(t - t0) >> 4];
    blk = blk < 0 ? 0 : blk;
    return (static_cast<int64_t>(blk) * 16 + (t & 15)) * p.G + g;
  };
  auto block_ok = [&](int t) -> bool { return !PAGED || sm_blk[(t - t0) >> 4] >= 0; };

  // K rows in the A-operand layout: token tbase + 16*tb + n, 16 bytes at dims kb*32 + grp*8
  auto issue_k = [&](int tbase, uint4 (&k)[2][KB]) {
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      int t = tbase + 16 * tb + n;
      t = t < t1 ? t : t0;
      const char* rp = kbase + row_of(t) * (2 * D) + grp * 16;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) k[tb][kb] = *reinterpret_cast<const uint4*>(rp + kb * 64);
    }
  };
  // V rows, coalesced, HBM -> LDS: instruction jj covers rows jj*RPI .. +RPI-1
  auto issue_v = [&](int tbase, char* buf) {
#pragma unroll
    for (int jj = 0; jj < NVL; ++jj) {
      int t = tbase + jj * RPI + lane / LPR;
      t = t < t1 ? t : t0;
      const char* src = vbase + row_of(t) * (2 * D) + (lane % LPR) * 16;
      __builtin_amdgcn_global_load_lds(src, (lds_ptr)(buf + jj * G::BLOCK), 16, 0, 0);
    }
  };

  char* vbuf[2] = {smem + (2 * wave) * G::kTileBytes, smem + (2 * wave + 1) * G::kTileBytes};
  uint4 kr[2][KB];
  int base = t0 + wave * TT;
  if (base < t1) {                    // tile 0 is requested before q
    issue_k(base, kr);
    issue_v(base, vbuf[0]);
  }

  // q as the B operand of the scores, staged once per workgroup in LDS: the
  // operand of lane (n, grp) for block (nb, kb) is dims kb*32 + grp*8 .. +7 of
  // head nb*16 + n, split into hi and lo.  Unconditional vector loads from a
  // valid head, then a select (a load under a per-lane branch would
  // serialise into one round trip per element).
  for (int idx = threadIdx.x; idx < NB * KB * 64; idx += 256) {
    const int ql_ = idx & 63, nbkb = idx >> 6;
    const int nb = nbkb / KB, kb = nbkb - nb * KB;
    const int h = nb * 16 + (ql_ & 15), gq = ql_ >> 4;
    const bool live = h < R;
    const float* src = p.q_rot + (static_cast<int64_t>(b) * p.H + hbase + (live ? h : 0)) * D;
    const float qs = live ? p.qscale : 0.f;
    const float4 x0 = *reinterpret_cast<const float4*>(src + kb * 32 + gq * 8);
    const float4 x1 = *reinterpret_cast<const float4*>(src + kb * 32 + gq * 8 + 4);
    const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    u16x8 hi, lo;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      unsigned short a, c;
      split_bf16(xv[j] * qs, a, c);
      hi[j] = a; lo[j] = c;
    }
    sm_q[(nbkb * 2 + 0) * 64 + ql_] = __builtin_bit_cast(uint4, hi);
    sm_q[(nbkb * 2 + 1) * 64 + ql_] = __builtin_bit_cast(uint4, lo);
  }
  __syncthreads();

  f32x4 acc[NB][CB];
  float m[NB], l[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    m[nb] = kNegInf; l[nb] = 0.f;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[nb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // One tile: `kr` holds its K rows, `vt` its V rows (being copied).  The
  // next tile's V copies go out first, into the other buffer; its K rows go
  // out right after this tile's score MFMAs have consumed `kr`.
  auto compute = [&](int tbase, uint4 (&kr)[2][KB], char* vt, char* vnext) {
    const int nbase = tbase + kWaves * TT;
    const bool more = nbase < t1;
    if (more) issue_v(nbase, vnext);
    const bool full = tbase + TT <= t1;
    bool blk_ok[2] = {true, true};
    if (PAGED) {
      blk_ok[0] = block_ok(tbase);
      blk_ok[1] = tbase + 16 < t1 ? block_ok(tbase + 16) : true;
    }
    // scores of the two 16-token halves
    f32x4 s[NB][2];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const bf16x8 a = __builtin_bit_cast(bf16x8, kr[h2][kb]);
          const bf16x8 qh = __builtin_bit_cast(bf16x8, sm_q[((nb * KB + kb) * 2 + 0) * 64 + lane]);
          const bf16x8 ql = __builtin_bit_cast(bf16x8, sm_q[((nb * KB + kb) * 2 + 1) * 64 + lane]);
          c = mfma(a, qh, c);
          c = mfma(a, ql, c);
        }
        s[nb][h2] = c;
      }
    if (more) issue_k(nbase, kr);        // K rows of the next tile, into the same registers

    bf16x8 ph[NB], pl[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float sv[8];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int t = tbase + 16 * h2 + 4 * grp + j;
          sv[h2 * 4 + j] = (t < t1 && blk_ok[h2]) ? s[nb][h2][j] : kNegInf;
        }
      float mt = sv[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) mt = fmaxf(mt, sv[j]);
      mt = fmaxf(mt, __shfl_xor(mt, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float mn = fmaxf(m[nb], mt);
      const float ref = mn == kNegInf ? 0.f : mn;
      if (__any(mn > m[nb])) {           // a running max moved: rescale
        const float alpha = exp2f(m[nb] - ref);
        l[nb] *= alpha;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) acc[nb][cb] *= alpha;
      }
      m[nb] = mn;
      u16x8 hi, lo;
      float ps = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float pj = exp2f(sv[j] - ref);
        ps += pj;
        unsigned short a, c;
        split_bf16(pj, a, c);
        hi[j] = a; lo[j] = c;
      }
      l[nb] += ps;
      ph[nb] = __builtin_bit_cast(bf16x8, hi);
      pl[nb] = __builtin_bit_cast(bf16x8, lo);
    }

    // this tile's V copies have landed: only the next tile's loads (V copies,
    // then K rows) may still be outstanding
    if (more) vmem_wait<G::NLOADS>();
    else vmem_wait<0>();
    if (!full || PAGED) {                // rows past the end or in a bad block become zeros
#pragma unroll
      for (int jj = 0; jj < NVL; ++jj) {
        const int r = jj * RPI + lane / LPR;
        const int t = tbase + r;
        if (!(t < t1 && blk_ok[r >> 4]))
          *reinterpret_cast<uint4*>(vt + G::at(r, (lane % LPR) * 16)) = make_uint4(0, 0, 0, 0);
      }
    }
    lds_fence();                         // the tile is visible to the whole wave

    // O^T[d][h] += V^T[d][t] P^T[t][h]; A row = dim 16*cb + n, tokens 16*(j/4) + 4*grp + j%4
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      u16x8 a;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int tok = 16 * (j >> 2) + 4 * grp + (j & 3);
        a[j] = *reinterpret_cast<const unsigned short*>(vt + G::at(tok, (16 * cb + n) * 2));
      }
      const bf16x8 av = __builtin_bit_cast(bf16x8, a);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        acc[nb][cb] = mfma(av, ph[nb], acc[nb][cb]);
        acc[nb][cb] = mfma(av, pl[nb], acc[nb][cb]);
      }
    }
    lds_fence();                         // reads done before this buffer is refilled
  };

  // the two V buffers alternate; K lives in one register set
  while (base < t1) {
    compute(base, kr, vbuf[0], vbuf[1]);
    base += kWaves * TT;
    if (base >= t1) break;
    compute(base, kr, vbuf[1], vbuf[0]);
    base += kWaves * TT;
  }

  // per-wave sums: the four lane groups of a head hold partial sums under one max
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    l[nb] += __shfl_xor(l[nb], 16);
    l[nb] += __shfl_xor(l[nb], 32);
  }

  // merge the waves through LDS, 16 heads at a time
  float* so = reinterpret_cast<float*>(smem);       // [kWaves][16][D]
  float* sm_m = so + kWaves * 16 * D;               // [kWaves][16]
  float* sm_l = sm_m + kWaves * 16;                 // [kWaves][16]
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int hb = nb * 16;
    const int nh = min(16, R - hb);
    if (nh <= 0) break;
    __syncthreads();                   // staging tiles / previous pass no longer read
    if (n < nh) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int j = 0; j < 4; ++j) so[(wave * 16 + n) * D + 16 * cb + 4 * grp + j] = acc[nb][cb][j];
      if (grp == 0) { sm_m[wave * 16 + n] = m[nb]; sm_l[wave * 16 + n] = l[nb]; }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < nh * D; idx += 256) {
      const int r = idx / D, d = idx - r * D;
      float M = sm_m[r];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm_m[w * 16 + r]);
      const float ref = M == kNegInf ? 0.f : M;
      float o = 0.f, sum = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float a = exp2f(sm_m[w * 16 + r] - ref);
        o += so[(w * 16 + r) * D + d] * a;
        sum += sm_l[w * 16 + r] * a;
      }
      const int h = hbase + hb + r;
      const float val = o / sum;
      const float lse2 = ref + log2f(sum);
      if (p.direct) {
        p.out[(static_cast<int64_t>(b) * p.H + h) * D + d] = val;
        if (d == 0 && p.lse) p.lse[static_cast<int64_t>(b) * p.H + h] = lse2 * 0.69314718055994531f;
      } else {
        const int64_t pr = (static_cast<int64_t>(b) * p.H + h) * p.n_splits + split;
        p.part_o[pr * D + d] = val;
        if (d == 0) p.part_lse[pr] = lse2;
      }
    }
  }
}

template <int D, int NB>
hipError_t launch_nb(const DecodeParams& p, bool paged, hipStream_t s) {
  const dim3 grid = p.grid_order == 0 ? dim3(p.n_splits, p.G, p.B)
                  : p.grid_order == 1 ? dim3(p.G, p.B, p.n_splits)
                                      : dim3(p.G, p.n_splits, p.B);
  if (paged) decode_mfma_kernel<D, NB, true><<<grid, 256, 0, s>>>(p);
  else decode_mfma_kernel<D, NB, false><<<grid, 256, 0, s>>>(p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeParams& p, bool paged, hipStream_t s) {
  return p.R <= 16 ? launch_nb<D, 1>(p, paged, s) : launch_nb<D, 2>(p, paged, s);
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeParams& p, bool paged, hipStream_t s) {
  if (p.chunk > kMfmaMaxChunk) return hipErrorInvalidValue;
  return p.D == 64 ? launch_d<64>(p, paged, s) : launch_d<128>(p, paged, s);
}

}  // namespace kvd
