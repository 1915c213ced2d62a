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
//           the A-operand layout (lane n of a 16-token half = token row
//           tile_row(n), 8 dims per lane), B = q.
//           q is fp32; it enters the bf16 product as q_hi + q_lo, two bf16
//           numbers whose sum is q to ~2^-17, as two MFMAs into one
//           accumulator, so scores keep near-fp32 accuracy while K is exact.
//           The q operands stay in registers for the whole split.
//   softmax the score output puts head h in lane h % 16 with tokens
//           16*tb + tile_row(4*(lane/16) + j); running max and sum per head live in
//           that lane, the tile max crosses the 4 lane groups with two
//           shuffles.  The running max is only moved (and the accumulators
//           rescaled) when a tile's max exceeds it by more than 2^8: until
//           then probabilities are taken against the stale max, which the
//           final normalisation by the sum cancels exactly.
//   P V     computed transposed, O^T[d][h] += sum_t V[t][d] P[h][t]: the B
//           operand P^T needs exactly the probabilities the lane holds (the
//           token order inside the contraction is free and chosen to match
//           the score layout), and each head's accumulators stay in its
//           lanes, so the rescale moves no data.  P is split hi + lo like q.
//           V^T is the A operand.  V rows travel HBM -> LDS directly
//           (buffer_load_dwordx4 ... lds, 16 bytes per lane, no registers): each
//           instruction lands 64 lanes x 16 bytes contiguously, rows in
//           order, and consecutive instructions are 32 bytes apart.  The
//           operand is read with gfx950's transposing ds_read_b64_tr_b16
//           (read_vt_tr), the tokens in tile_row order so that each 16-lane
//           group reads rows of four different copy instructions (banks 8
//           apart).  Rows past the end of the sequence or in an invalid
//           block are read out of range, and are also zeroed in LDS after
//           the copy in the tiles that have them (stale LDS may hold NaN and
//           0 * NaN is NaN).
//
// Software pipeline: while tile i is computed, tile i+1 is in flight -- its V
// rows into the second of two LDS buffers from the start of tile i, its K
// rows into the K registers as soon as tile i's score MFMAs have read them --
// so a wave keeps up to 16 KB of loads outstanding while it works.
// Vector-memory loads complete in issue order, so "at most N outstanding"
// (s_waitcnt vmcnt(N), N = the loads of one tile) says tile i has landed.
// The LDS reads and writes of the staged tiles are issued from inline
// assembly on purpose: the compiler cannot tell that they do not touch the
// buffer an HBM -> LDS copy is still filling, and would otherwise wait for
// every outstanding copy before each of them, which serialises the pipeline.
// Their ordering against the copies is the explicit vmcnt wait above.
// The copies are MUBUF (buffer) loads rather than global ones: the compiler
// treats a pending global HBM -> LDS copy like a FLAT access and then turns
// its own wait for the K registers into a wait for everything.
// Paged block ids are held in registers (lane j = j-th block this wave
// visits) and broadcast with readlane, so no table or LDS load sits between
// two tiles' loads.  Waves of a workgroup take interleaved tiles of the
// split and merge their (m, l, O) through LDS at the end.
#include "mfma_tile.h"

namespace kvd {
namespace {

using namespace mt;

// block ids per wave held in registers: 64 per VGPR
constexpr int kBlkRegs = (kMfmaMaxChunk / 16 / kMfmaWaves + 63) / 64;

// LDS of a workgroup: two staged V tiles per wave, reused for the merge
template <int D>
constexpr int smem_bytes() {
  constexpr int stage = kMfmaWaves * 2 * Geo<D>::kTileBytes;
  constexpr int merge = merge_bytes<D>();
  return stage > merge ? stage : merge;
}

// LDS of the fused step's rotation factors: wave 0's second V buffer, free
// until that wave requests its second tile (after a barrier)
typedef __attribute__((address_space(3))) double lds_f64;

// One (sequence b, KV head g, split) unit computed by the whole workgroup:
// the waves take interleaved tiles of the split, merge through LDS and
// write the split's normalised output and log-sum-exp (or the final output
// when there is a single split).  FUSED (the decode step in one launch, T
// new tokens at positions P .. P + T - 1): q is rotated here from the raw
// q, and each workgroup whose split holds window tokens (the last split
// also those past the host bound) appends their k and v first.
template <int D, int NB, bool PAGED, bool FUSED = false>
__device__ __forceinline__ void run_split(const DecodeParams& p, char* smem, int b, int g, int split) {
  using G = Geo<D>;
  constexpr int KB = G::KB, CB = G::CB, TT = G::TT, LPR = G::LPR, RPI = G::RPI, NVL = G::NVL;
  constexpr int kWaves = kMfmaWaves;
  static_assert(TT == 32 && NB >= 1 && NB <= 2, "tile shape");
  const int R = p.R;
  const int RT = R * p.T;             // tile columns: the query rows of this KV head
  const int raw_len = scalar_load_i32(p.seq_lens + b);   // FUSED: the first new token's position
  const int L = attended_len(p, len_of(p, raw_len));
  const int t0 = split_start(p, split);
  if (t0 >= L) {
    if (p.direct && split == 0) {     // empty sequence: out = 0, lse = -inf
      for (int idx = threadIdx.x; idx < RT * D; idx += 256) {
        const int r = idx / D, d = idx - r * D;
        const int64_t row = query_row(p, b, g, r);
        p.out[row * D + d] = 0.f;
        if (d == 0 && p.lse) p.lse[row] = kNegInf;
      }
    }
    return;
  }
  const int t1 = min(t0 + split_size(p, split), L);
  // several new tokens: column c (token c / R) sees the tokens below
  // L - T + 1 + c / R; tiles reaching past win need the per-column bound
  const int win = L - p.T + 1;
  int cbound[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int c = nb * 16 + (threadIdx.x & 15);
    cbound[nb] = c < RT ? win + c / R : L;
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, grp = lane >> 4;
  // bytes between consecutive tokens of one KV head, and the start of this
  // (sequence, KV head) -- of KV head g of the pool when paged
  const int64_t rs = static_cast<int64_t>(p.G) * (2 * D);
  const int64_t head0 = (PAGED ? 0 : static_cast<int64_t>(b) * p.max_seq_len * rs) +
                        static_cast<int64_t>(g) * (2 * D);
  const char* kbase = static_cast<const char*>(p.k) + head0;
  const char* vbase = static_cast<const char*>(p.v) + head0;

  // q operands, requested first: lane (n, grp) of block (nb, kb) holds dims
  // kb*32 + grp*8 .. +7 of head nb*16 + n.  Unconditional vector loads from a
  // valid head, then a select (a load under a per-lane branch would
  // serialise into one round trip per element).  With two column blocks the
  // rows are loaded once per workgroup and staged in LDS (QStage).
  float4 qraw[NB][KB][2];
  QStage<D> qst;
  // FUSED: the raw q (bf16), rotated once the factors are in LDS; with two
  // column blocks in QStage's layout (4 dims of rows 8w + i RPI + lane/LPR)
  using QS = QStage<D>;
  uint4 qin[FUSED && NB == 1 ? KB : 1];
  uint2 qin2[FUSED && NB == 2 ? QS::NI : 1];
  if constexpr (NB == 2 && FUSED) {
#pragma unroll
    for (int i = 0; i < QS::NI; ++i) {
      const int r = 8 * wave + i * QS::RPI + lane / QS::LPR;
      qin2[i] = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p.q_in) +
                                                query_row(p, b, g, r < RT ? r : 0) * D +
                                                4 * (lane % QS::LPR));
    }
  } else if constexpr (NB == 2) {
    qst.load(p, b, g, RT, wave, lane);
  } else if constexpr (FUSED) {
    const int h = n;
    const uint16_t* src =
        static_cast<const uint16_t*>(p.q_in) + query_row(p, b, g, h < RT ? h : 0) * D + grp * 8;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) qin[kb] = *reinterpret_cast<const uint4*>(src + kb * 32);
  } else {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int h = nb * 16 + n;
      const float* src = p.q_rot + query_row(p, b, g, h < RT ? h : 0) * D + grp * 8;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        qraw[nb][kb][0] = *reinterpret_cast<const float4*>(src + kb * 32);
        qraw[nb][kb][1] = *reinterpret_cast<const float4*>(src + kb * 32 + 4);
      }
    }
  }

  // paged: the ids of the blocks this wave visits, lane j of register c =
  // the wave's (64c + j)-th block = split block 8*(i/2) + 2*wave + i%2 with
  // i = 64c + j (tile i/2 of the wave, half i%2); ids outside the pool
  // become -1
  int blkv[PAGED ? kBlkRegs : 1];
  if (PAGED) {
    const int nblk = (t1 - t0 + 15) >> 4;
#pragma unroll
    for (int c = 0; c < kBlkRegs; ++c) {
      const int i = c * 64 + lane;
      int sb = 8 * (i >> 1) + 2 * wave + (i & 1);
      sb = sb < nblk ? sb : nblk - 1;
      blkv[c] = paged_group(p, b, (t0 >> 4) + sb);
    }
  }
  // block ids (wave-uniform) of the two 16-token halves of the wave's tile kt
  auto tile_blocks = [&](int kt, int (&blk)[2]) {
    if (!PAGED) { blk[0] = blk[1] = 0; return; }
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const int i = 2 * kt + tb;
      int v = blkv[0];
#pragma unroll
      for (int c = 1; c < kBlkRegs; ++c) v = (i >> 6) == c ? blkv[c] : v;
      blk[tb] = __builtin_amdgcn_readlane(v, i & 63);
    }
  };

  // Each 16-token half of a tile is read through two buffer descriptors
  // (K and V) that start at the half's first token row and end at the last
  // valid one: tokens at or past the end of the split, and every token of an
  // invalid block, are out of range and read as zeros without touching
  // memory (the last tile may reach past S_max).  Per-lane offsets are then
  // the same for every tile.
  struct TileSrc { rsrc_t k[2], v[2]; };
  auto tile_src = [&](int tbase, const int (&blk)[2]) {
    TileSrc ts;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int lo = tbase + 16 * h;
      int rows = t1 - lo;
      rows = rows < 0 ? 0 : (rows > 16 ? 16 : rows);
      int64_t off;
      if (PAGED) {
        if (blk[h] < 0) rows = 0;
        off = static_cast<int64_t>(blk[h] < 0 ? 0 : blk[h]) * 16 * rs;
      } else {
        off = static_cast<int64_t>(lo) * rs;
      }
      // wave-uniform by construction; readfirstlane keeps the descriptor in
      // scalar registers (a VALU clamp would otherwise make it look divergent)
      rows = __builtin_amdgcn_readfirstlane(rows);
      const uint32_t bytes = static_cast<uint32_t>(rows) * static_cast<uint32_t>(rs);
      ts.k[h] = make_rsrc(kbase + off, bytes);
      ts.v[h] = make_rsrc(vbase + off, bytes);
    }
    return ts;
  };
  // K rows in the A-operand layout: row n of half tb, 16 bytes at dims
  // kb*32 + grp*8
  const uint32_t koff = static_cast<uint32_t>(tile_row(n) * rs + grp * 16);
  auto issue_k = [&](const TileSrc& ts, uint4 (&k)[2][KB]) {
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        k[tb][kb] = load16(ts.k[tb], koff + kb * 64);
  };
  // V rows, coalesced, HBM -> LDS: instruction jj covers tile rows
  // jj*RPI .. +RPI-1, i.e. rows (jj*RPI) % 16 + lane/LPR of half jj*RPI/16
  const uint32_t vlane = static_cast<uint32_t>((lane / LPR) * rs + (lane % LPR) * 16);
  auto issue_v = [&](const TileSrc& ts, lds_char* buf) {
#pragma unroll
    for (int jj = 0; jj < NVL; ++jj) {
      const uint32_t off = vlane + static_cast<uint32_t>(((jj * RPI) % 16) * rs);
      copy16_to_lds(ts.v[(jj * RPI) / 16], buf + jj * G::BLOCK, off);
    }
  };

  lds_char* const stage = (lds_char*)(smem);
  lds_char* vbuf[2] = {stage + (2 * wave) * G::kTileBytes, stage + (2 * wave + 1) * G::kTileBytes};
  // this lane's address for read_vt_tr: row tile_row(4 grp + n / 4), dims 4 (n % 4) ..
  const uint32_t vrd_off = G::at(tile_row(4 * grp + n / 4), 8 * (n % 4));
  const uint32_t vrd[2] = {lds_addr(vbuf[0]) + vrd_off, lds_addr(vbuf[1]) + vrd_off};
  constexpr int kVHalf = (16 / RPI) * G::BLOCK;     // rows r -> r + 16
  uint4 kr[2][KB];
  int blk_cur[2];
  int base = t0 + wave * TT;
  tile_blocks(0, blk_cur);
  // FUSED: a workgroup whose split holds window tokens appends them (the
  // last split also those at or past the host bound), and must not request
  // its first tile before that; wave-uniform
  const int P0 = raw_len;
  const bool last_split = split == split_count(p, L) - 1;
  const int app_lo = P0 > t0 ? P0 : t0;
  const int64_t win_end = static_cast<int64_t>(P0) + p.T;
  const int64_t split_end = static_cast<int64_t>(t0) + split_size(p, split);
  const int app_hi = static_cast<int>(last_split || win_end < split_end ? win_end : split_end);
  const bool appender = FUSED && app_lo < app_hi;
  if (!appender) {
    // issued on every path (a wave without tiles gets empty descriptors and
    // reads nothing), so the wait for the q loads above stays partial
    const TileSrc ts = tile_src(base, blk_cur);
    issue_k(ts, kr);
    issue_v(ts, vbuf[0]);
  }
  if constexpr (FUSED) {
    // RoPE factors of each new token's position (token t at P0 + t), in
    // fp64 as the append kernel computes them, into LDS: token t's table in
    // wave t % 4's second V buffer (past the 8 q rows QStage keeps there
    // with two column blocks), t / 4 tables in (up to 16 tokens)
    static_assert((NB == 2 ? 8 * QS::ROW : 0) + 4 * D * 8 <= G::kTileBytes,
                  "four factor tables beside the staged q rows");
    auto fac = [&](int t) {
      return reinterpret_cast<lds_f64*>(stage + (2 * (t & 3) + 1) * G::kTileBytes +
                                        (NB == 2 ? 8 * QS::ROW : 0) + (t >> 2) * D * 8);
    };
    {
      // thread (t, i): theta_i once, then tokens t, t + 256 / (D/2), ...
      const int i = threadIdx.x % (D / 2);
      const double theta = pow(p.rope_base, -2.0 * i / D);
      for (int t = threadIdx.x / (D / 2); t < p.T; t += 256 / (D / 2)) {
        double sv, cv;
        sincos(static_cast<double>(static_cast<int64_t>(P0) + t) * theta, &sv, &cv);
        fac(t)[i] = cv;
        fac(t)[D / 2 + i] = sv;
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const bool inter = p.rope_style != KVD_ROPE_HALF;
    if (appender) {
      // each of its window tokens: k_new rotated and rounded once to bf16,
      // v_new copied, into the token's cache slot (skipped outside the
      // cache); the stores land before any wave requests a tile, and the
      // tiles that hold the tokens read them.  Item c < D/8 of a token
      // rotates 4 pairs of k: elements 8c .. 8c+7 (interleaved) or
      // 4c .. 4c+3 with 4c+D/2 .. (half), pair k using factor 4c + k; item
      // D/8 + c copies v elements 8c .. 8c+7 (16-byte accesses)
      constexpr int N8 = D / 8;
      for (int idx = threadIdx.x; idx < (app_hi - app_lo) * 2 * N8; idx += 256) {
        const int pos = app_lo + idx / (2 * N8), it = idx % (2 * N8), t = pos - P0;
        if (pos < 0 || pos >= p.max_seq_len) continue;
        int64_t row = -1;
        if (PAGED) {
          const int grp16 = paged_group(p, b, pos >> 4);
          if (grp16 >= 0) row = (static_cast<int64_t>(grp16) * 16 + (pos & 15)) * p.G + g;
        } else {
          row = (static_cast<int64_t>(b) * p.max_seq_len + pos) * p.G + g;
        }
        if (row < 0) continue;
        const int64_t src = ((static_cast<int64_t>(b) * p.T + t) * p.G + g) * D;
        if (it < N8) {
          const uint16_t* kn = static_cast<const uint16_t*>(p.k_new) + src;
          uint16_t* kc = static_cast<uint16_t*>(const_cast<void*>(p.k)) + row * D;
          const lds_f64* const fc = fac(t);
          // the 4 pairs as (a, c) -> (a cos - c sin, a sin + c cos)
          auto rot = [&](float a, float c, int f, uint16_t& ra, uint16_t& rc) {
            const double cf = fc[f], sf = fc[D / 2 + f];
            ra = double_to_bf16_rne(static_cast<double>(a) * cf - static_cast<double>(c) * sf);
            rc = double_to_bf16_rne(static_cast<double>(a) * sf + static_cast<double>(c) * cf);
          };
          if (inter) {
            const uint4 w = *reinterpret_cast<const uint4*>(kn + 8 * it);
            const uint32_t wi[4] = {w.x, w.y, w.z, w.w};
            uint32_t wo[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              uint16_t ra, rc;
              rot(bf16lo(wi[k]), bf16hi(wi[k]), 4 * it + k, ra, rc);
              wo[k] = static_cast<uint32_t>(ra) | (static_cast<uint32_t>(rc) << 16);
            }
            *reinterpret_cast<uint4*>(kc + 8 * it) = make_uint4(wo[0], wo[1], wo[2], wo[3]);
          } else {
            const uint2 x = *reinterpret_cast<const uint2*>(kn + 4 * it);
            const uint2 y = *reinterpret_cast<const uint2*>(kn + 4 * it + D / 2);
            const float xa[4] = {bf16lo(x.x), bf16hi(x.x), bf16lo(x.y), bf16hi(x.y)};
            const float ya[4] = {bf16lo(y.x), bf16hi(y.x), bf16lo(y.y), bf16hi(y.y)};
            uint16_t ra[4], rc[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) rot(xa[k], ya[k], 4 * it + k, ra[k], rc[k]);
            *reinterpret_cast<uint2*>(kc + 4 * it) =
                make_uint2(ra[0] | (static_cast<uint32_t>(ra[1]) << 16),
                           ra[2] | (static_cast<uint32_t>(ra[3]) << 16));
            *reinterpret_cast<uint2*>(kc + 4 * it + D / 2) =
                make_uint2(rc[0] | (static_cast<uint32_t>(rc[1]) << 16),
                           rc[2] | (static_cast<uint32_t>(rc[3]) << 16));
          }
        } else {
          const int c = it - N8;
          *reinterpret_cast<uint4*>(static_cast<uint16_t*>(const_cast<void*>(p.v)) + row * D +
                                    8 * c) =
              *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.v_new) + src + 8 * c);
        }
      }
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
      const TileSrc ts = tile_src(base, blk_cur);
      issue_k(ts, kr);
      issue_v(ts, vbuf[0]);
    }
    if constexpr (NB == 2) {
      // rotate this lane's 4 dims (4c .. 4c+3, c = lane % LPR) of each of
      // its rows: interleaved pairs sit in them; the half pair of dim d <
      // D/2 is d + D/2, held by the lane LPR/2 apart in the same row
      const int c = lane % QS::LPR;
#pragma unroll
      for (int i = 0; i < QS::NI; ++i) {
        const int r = 8 * wave + i * QS::RPI + lane / QS::LPR;
        const lds_f64* const fcos = fac((r < RT ? r : 0) / R);
        const lds_f64* const fsin = fcos + D / 2;
        float x[4] = {bf16lo(qin2[i].x), bf16hi(qin2[i].x), bf16lo(qin2[i].y), bf16hi(qin2[i].y)};
        if (inter) {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int f = 2 * c + j;
            const double a = x[2 * j], cc = x[2 * j + 1];
            const double cf = fcos[f], sf = fsin[f];
            x[2 * j] = static_cast<float>(a * cf - cc * sf);
            x[2 * j + 1] = static_cast<float>(a * sf + cc * cf);
          }
        } else {
          const bool low = c < QS::LPR / 2;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float other = __shfl_xor(x[e], QS::LPR / 2);
            const int f = 4 * (c % (QS::LPR / 2)) + e;
            const double own = x[e], par = other;
            const double cf = fcos[f], sf = fsin[f];
            x[e] = low ? static_cast<float>(own * cf - par * sf)
                       : static_cast<float>(par * sf + own * cf);
          }
        }
        qst.v[i] = make_float4(x[0], x[1], x[2], x[3]);
        if (p.q_rot_out && split == 0 && r < RT)
          *reinterpret_cast<float4*>(p.q_rot_out + query_row(p, b, g, r) * D + 4 * c) = qst.v[i];
      }
    } else {
    // rotate this lane's q dims (pairs 2i, 2i+1, or i and i + D/2 held in
    // blocks kb and kb + KB/2), fp64, rounded once to fp32 as q_rot; the
    // lane's row n is token n / R
    const lds_f64* const fcos = fac((n < RT ? n : 0) / R);
    const lds_f64* const fsin = fcos + D / 2;
    float qv[KB][8];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const uint32_t w[4] = {qin[kb].x, qin[kb].y, qin[kb].z, qin[kb].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        qv[kb][2 * j] = bf16lo(w[j]);
        qv[kb][2 * j + 1] = bf16hi(w[j]);
      }
    }
    if (inter) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int f = kb * 16 + grp * 4 + j;
          const double a = qv[kb][2 * j], c = qv[kb][2 * j + 1];
          const double cf = fcos[f], sf = fsin[f];
          qv[kb][2 * j] = static_cast<float>(a * cf - c * sf);
          qv[kb][2 * j + 1] = static_cast<float>(a * sf + c * cf);
        }
    } else {
#pragma unroll
      for (int kb = 0; kb < KB / 2; ++kb)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int f = kb * 32 + grp * 8 + e;
          const double a = qv[kb][e], c = qv[kb + KB / 2][e];
          const double cf = fcos[f], sf = fsin[f];
          qv[kb][e] = static_cast<float>(a * cf - c * sf);
          qv[kb + KB / 2][e] = static_cast<float>(a * sf + c * cf);
        }
    }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      qraw[0][kb][0] = make_float4(qv[kb][0], qv[kb][1], qv[kb][2], qv[kb][3]);
      qraw[0][kb][1] = make_float4(qv[kb][4], qv[kb][5], qv[kb][6], qv[kb][7]);
    }
    // q_rot for the caller, written once per (sequence, KV head)
    if (p.q_rot_out && split == 0 && n < RT) {
      float* dst = p.q_rot_out + query_row(p, b, g, n) * D + grp * 8;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        *reinterpret_cast<float4*>(dst + kb * 32) = qraw[0][kb][0];
        *reinterpret_cast<float4*>(dst + kb * 32 + 4) = qraw[0][kb][1];
      }
    }
    }
    // every wave has read the factors before wave 0 copies its second tile
    // over them (with two column blocks also before QStage's rows are
    // written beside them)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }

  if constexpr (NB == 2) {
    const uint32_t st = lds_addr(stage);
    qst.publish(st, G::kTileBytes, wave, lane);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int h = nb * 16 + n;
      const uint32_t a = QStage<D>::row_addr(st, G::kTileBytes, h < RT ? h : 0) + 32 * grp;
      static_for<KB>([&](auto kbc) {
        constexpr int kb = decltype(kbc)::value;
        read_b128x2<128 * kb>(a, qraw[nb][kb][0], qraw[nb][kb][1]);
      });
    }
    __builtin_amdgcn_s_barrier();      // every wave's q read before the rows are reused
  }

  // q * scale * log2(e) as bf16 hi + lo (heads >= n_rep get zeros)
  bf16x8 qh[NB][KB], ql[NB][KB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float qs = nb * 16 + n < RT ? p.qscale : 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const float4 x0 = qraw[nb][kb][0], x1 = qraw[nb][kb][1];
      const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      u16x8 hi, lo;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        unsigned short a, c;
        split_bf16(xv[j] * qs, a, c);
        hi[j] = a; lo[j] = c;
      }
      qh[nb][kb] = __builtin_bit_cast(bf16x8, hi);
      ql[nb][kb] = __builtin_bit_cast(bf16x8, lo);
    }
  }

  f32x4 acc[NB][CB];
  float m[NB], l[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    m[nb] = kNegInf; l[nb] = 0.f;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[nb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // The pieces of one tile's work.  Scores of the two 16-token halves from
  // the K registers:
  auto scores = [&](const uint4 (&k)[2][KB], f32x4 (&sc)[NB][2]) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const bf16x8 a = __builtin_bit_cast(bf16x8, k[h2][kb]);
          c = mfma(a, qh[nb][kb], c);
          c = mfma(a, ql[nb][kb], c);
        }
        sc[nb][h2] = c;
      }
  };
  // Online softmax of a tile's scores (tokens at or past the end, in a bad
  // block, or past a column's bound excluded when `masked`): moves the
  // running max when needed and returns the probabilities as bf16 hi + lo.
  auto softmax = [&](f32x4 (&sc)[NB][2], int tbase, bool masked, bool ok0, bool ok1,
                     bf16x8 (&ph)[NB], bf16x8 (&pl)[NB]) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float sv[8];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int j = 0; j < 4; ++j) sv[h2 * 4 + j] = sc[nb][h2][j];
      if (masked) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int t = tbase + 16 * h2 + tile_row(4 * grp + j);
            const bool ok = h2 == 0 ? ok0 : ok1;
            if (!(t < t1 && ok && t < cbound[nb])) sv[h2 * 4 + j] = kNegInf;
          }
      }
      float mt = sv[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) mt = fmaxf(mt, sv[j]);
      mt = fmaxf(mt, __shfl_xor(mt, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      if (__builtin_expect(__any(mt > m[nb] + kRescaleSlack), 0)) {   // a running max moves: rescale
        const float mn = fmaxf(m[nb], mt);
        const float alpha = mn == kNegInf ? 1.f : __builtin_amdgcn_exp2f(m[nb] - mn);
        l[nb] *= alpha;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) acc[nb][cb] *= alpha;
        m[nb] = mn;
      }
      const float ref = m[nb] == kNegInf ? 0.f : m[nb];
      u16x8 hi, lo;
      float ps = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float pj = __builtin_amdgcn_exp2f(sv[j] - ref);
        ps += pj;
        unsigned short a, c;
        split_bf16(pj, a, c);
        hi[j] = a; lo[j] = c;
      }
      l[nb] += ps;
      ph[nb] = __builtin_bit_cast(bf16x8, hi);
      pl[nb] = __builtin_bit_cast(bf16x8, lo);
    }
  };
  // Staged V rows past the end or in a bad block become zeros (after the
  // tile's copies have landed; stale LDS may hold NaN and 0 * NaN is NaN).
  auto zero_rows = [&](uint32_t vt, int tbase, bool ok0, bool ok1) {
#pragma unroll
    for (int jj = 0; jj < NVL; ++jj) {
      const int r = jj * RPI + lane / LPR;
      const bool ok = (jj * RPI) / 16 == 0 ? ok0 : ok1;
      if (!(tbase + r < t1 && ok)) lds_zero16(vt + jj * G::BLOCK + lane * 16);
    }
  };
  // O^T[d][h] += V^T[d][t] P^T[t][h]; A row = dim 16*cb + n, tokens
  // 16*(j/4) + tile_row(4*grp + j%4) (transposing LDS reads at `vaddr`,
  // this lane's read address in the staged tile)
  auto pv = [&](uint32_t vaddr, const bf16x8 (&ph)[NB], const bf16x8 (&pl)[NB]) {
    static_for<CB>([&](auto cbc) {
      constexpr int cb = decltype(cbc)::value;
      const bf16x8 av = read_vt_tr<32 * cb, kVHalf>(vaddr);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        acc[nb][cb] = mfma(av, ph[nb], acc[nb][cb]);
        acc[nb][cb] = mfma(av, pl[nb], acc[nb][cb]);
      }
    });
  };

  {
    // One tile (the wave's kt-th): `kr` holds its K rows, buffer `cur` its V
    // rows (being copied), `blk` its block ids.  The next tile's V copies go
    // out first, into the other buffer; its K rows go out right after this
    // tile's score MFMAs have consumed `kr`.  `more` (a constant at each
    // call) says whether there is a next tile: the loads are then issued on
    // every path, so the compiler's own wait for `kr` counts them and stays
    // partial.
    auto compute = [&](int kt, int tbase, int (&blk)[2], int cur, const bool more) {
      const int nbase = tbase + kWaves * TT;
      int blk_next[2];
      tile_blocks(kt + 1, blk_next);
      const TileSrc ns = tile_src(nbase, blk_next);
      if (more) {
        issue_v(ns, vbuf[cur ^ 1]);
        // keep the copies ahead of the score MFMAs, whose wait for `kr` may
        // then leave them outstanding
        __builtin_amdgcn_sched_barrier(0);
      }
      const bool full = tbase + TT <= t1;
      const bool ok0 = !PAGED || blk[0] >= 0;
      const bool ok1 = !PAGED || blk[1] >= 0;
      const bool masked = !full || !ok0 || !ok1 || tbase + TT > win;      // wave-uniform
      f32x4 sc[NB][2];
      scores(kr, sc);
      if (more) issue_k(ns, kr);          // K rows of the next tile, into the same registers
      bf16x8 ph[NB], pl[NB];
      softmax(sc, tbase, masked, ok0, ok1, ph, pl);
      // this tile's V copies have landed: only the next tile's loads (V
      // copies, then K rows) may still be outstanding
      if (more) vmem_wait<G::NLOADS>();
      else vmem_wait<0>();
      if (masked) zero_rows(lds_addr(vbuf[cur]), tbase, ok0, ok1);
      pv(vrd[cur], ph, pl);
      blk[0] = blk_next[0];
      blk[1] = blk_next[1];
    };

    // the two V buffers alternate; K lives in one register set; the wave's
    // last tile is peeled off (no next tile to request)
    if (base < t1) {
      int kt = 0, cur = 0;
      while (base + kWaves * TT < t1) {
        compute(kt, base, blk_cur, cur, true);
        base += kWaves * TT;
        ++kt;
        cur ^= 1;
      }
      compute(kt, base, blk_cur, cur, false);
    }
  }
  // a wave without tiles still has its (empty) copies outstanding: they
  // write zeros into its staging buffers, which the merge below reuses
  vmem_wait<0>();

  // per-wave sums: the four lane groups of a head hold partial sums under one max
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    l[nb] += __shfl_xor(l[nb], 16);
    l[nb] += __shfl_xor(l[nb], 32);
  }

  // merge the waves through LDS, 16 rows at a time
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int nh = min(16, RT - nb * 16);
    if (nh <= 0) break;
    merge_waves<D>(p, smem, b, g, split, nb * 16, nh, acc[nb], m[nb], l[nb], 1.f);
  }
}

// One workgroup per unit, dispatched by the hardware in the planner's order.
// Up to 16 query rows per KV head:
template <int D, bool PAGED, bool FUSED>
__global__ __launch_bounds__(256) void decode_mfma_kernel(DecodeParams p) {
  __shared__ __align__(16) char smem[smem_bytes<D>()];
  Unit u;
  if (!unit_at(p, u)) return;
  run_split<D, 1, PAGED, FUSED>(p, smem, u.b, u.g, u.split);
}
// 17 to 32 query rows per KV head (two column blocks): left to itself the
// compiler splits the accumulators into AGPRs and needs 295 registers per
// lane at D = 128, one workgroup per CU; held to 256 it fits them in VGPRs
// without spilling, and two workgroups share a CU.
template <int D, bool PAGED, bool FUSED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void decode_mfma_kernel_wide(DecodeParams p) {
  __shared__ __align__(16) char smem[smem_bytes<D>()];
  Unit u;
  if (!unit_at(p, u)) return;
  run_split<D, 2, PAGED, FUSED>(p, smem, u.b, u.g, u.split);
}

template <int D, int NB>
hipError_t launch_nb(const DecodeParams& p, bool paged, const Launch& l) {
  void (*k)(DecodeParams) =
      NB == 1 ? (p.len_bias ? (paged ? decode_mfma_kernel<D, true, true> : decode_mfma_kernel<D, false, true>)
                            : (paged ? decode_mfma_kernel<D, true, false> : decode_mfma_kernel<D, false, false>))
              : (p.len_bias ? (paged ? decode_mfma_kernel_wide<D, true, true>
                                     : decode_mfma_kernel_wide<D, false, true>)
                            : (paged ? decode_mfma_kernel_wide<D, true, false>
                                     : decode_mfma_kernel_wide<D, false, false>));
  return launch_kernel(k, split_grid(p), dim3(256), l, p);
}

template <int D>
hipError_t launch_d(const DecodeParams& p, bool paged, const Launch& l) {
  return p.R * p.T <= 16 ? launch_nb<D, 1>(p, paged, l) : launch_nb<D, 2>(p, paged, l);
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeParams& p, bool paged, const Launch& l) {
  if (p.chunk > kMfmaMaxChunk || p.chunk % 16 != 0 || p.chunk2 > p.chunk || p.chunk2 < 16 ||
      p.chunk2 % 16 != 0 || p.n_big < 0 || p.n_big > p.n_splits || p.T < 1 || p.R * p.T > 32 ||
      p.row_groups > 1)
    return hipErrorInvalidValue;
  // the fused step: lengths positions + T, up to 16 new tokens (four factor
  // tables per wave buffer), its inputs given
  if (p.len_bias && (p.len_bias != p.T || p.T > 16 || !p.q_in || !p.k_new || !p.v_new))
    return hipErrorInvalidValue;
  return p.D == 64 ? launch_d<64>(p, paged, l) : launch_d<128>(p, paged, l);
}

}  // namespace kvd
