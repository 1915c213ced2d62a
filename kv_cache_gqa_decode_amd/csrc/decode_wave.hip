// Persistent split-K decode attention on the matrix cores, one wave per
// (sequence, KV head, split) unit, with the next unit's loads issued while
// the current one finishes (bf16 KV, D in {64, 128}, up to 32 query heads
// per KV head).
//
// What is computed is the same as in the other kernels -- per (b, h) the
// softmax(q K^T * scale) V over the sequence's L_b cached tokens,
// "Transformer推理核心：KV Cache、GQA与RoPE原理与工程实践" §2.1/§4.2, the n_rep
// query heads of a KV head sharing every K/V tile (§2.2 of the same page) --
// and so is the per-tile arithmetic of mfma_tile.h: MFMA scores against q
// split into bf16 hi + lo, online softmax with a lazily moved running max,
// P V computed transposed from a V tile staged in LDS.
//
// What differs is how the units reach the compute units.  With one
// workgroup per unit, every unit pays a start (its length, q, the first
// tile's round trip) and an end (a cross-wave merge) during which its slot
// streams nothing, and the hardware's oldest-first issue makes the second
// workgroup on a compute unit run up to half again as long as the first, so
// the last round of units drags on.  Here a grid sized to what the device
// holds at once keeps running: each wave takes the next unit number from an
// atomic counter in the workspace and computes that unit alone, tile after
// tile, writing its normalised partial output and log-sum-exp from
// registers (no merge, no barrier).  The unit after the current one is
// claimed when the current one starts; at the current unit's last tile,
// right after its score MFMAs, the wave decodes that next unit and issues
// its q loads and first K/V tile into the free V buffer before it finishes
// the last tile's softmax and P V and writes its result, so the stream of
// loads does not stop between units.  Faster waves simply take more units.
//
// The last wave to leave puts the two counters back to zero: they must be
// zero before the first call on a workspace and are zero after every call.
// Unit numbers compare unsigned, so counters that do not start at zero can
// only make waves leave early, never index outside the batch.
#include "mfma_tile.h"

namespace kvd {
namespace {

using namespace mt;

// block ids of one unit held in registers: 64 per VGPR
constexpr int kUnitBlkRegs = kWaveMaxChunk / 16 / 64;

template <int D, int NB, bool PAGED>
__global__ __launch_bounds__(256) void decode_wave_kernel(DecodeParams p) {
  using G = Geo<D>;
  constexpr int KB = G::KB, CB = G::CB, TT = G::TT, LPR = G::LPR, RPI = G::RPI, NVL = G::NVL;
  static_assert(TT == 32 && NB >= 1 && NB <= 2, "tile shape");
  __shared__ __align__(16) char smem[kMfmaWaves * 2 * G::kTileBytes];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, grp = lane >> 4;
  const int R = p.R;
  // bytes between consecutive tokens of one KV head
  const int64_t rs = static_cast<int64_t>(p.G) * (2 * D);
  lds_char* const stage = (lds_char*)(smem);
  lds_char* vbuf[2] = {stage + (2 * wave) * G::kTileBytes, stage + (2 * wave + 1) * G::kTileBytes};
  const uint32_t vrd[2] = {lds_addr(vbuf[0]) + G::at(4 * grp, 2 * n),
                           lds_addr(vbuf[1]) + G::at(4 * grp, 2 * n)};
  // per-lane byte offsets inside a 16-token half: K in the A-operand layout
  // (row n, 16 bytes at dims kb*32 + grp*8), V rows for the LDS copies
  const uint32_t koff = static_cast<uint32_t>(n * rs + grp * 16);
  const uint32_t vlane = static_cast<uint32_t>((lane / LPR) * rs + (lane % LPR) * 16);
  typedef __attribute__((address_space(1))) uint32_t global_u32;
  global_u32* const ctr = (global_u32*)(p.counters);

  // lane 0 takes the next unit number (the value lives in lane 0 only)
  auto claim = [&]() -> int {
    int v = 0;
    if (lane == 0)
      v = static_cast<int>(__hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    return v;
  };

  // ------------------------------------------------------------ one unit
  struct Unit_ {
    int b, g, split, hbase, t0, t1;
    const char* kbase;
    const char* vbase;
  };
  // Decode unit `item`; false when it holds no token (for a sequence with no
  // token at all, split 0 with a single split writes the empty result).
  auto open_unit = [&](int item, Unit_& u) -> bool {
    const Unit c = unit_of_item(p, item);
    int L = scalar_load_i32(p.seq_lens + c.b);
    L = L < 0 ? 0 : (L > p.max_len_host ? p.max_len_host : L);
    u.b = c.b; u.g = c.g; u.split = c.split;
    u.hbase = c.g * R;
    u.t0 = split_start(p, c.split);
    if (u.t0 >= L) {
      if (p.direct && c.split == 0) {
        for (int idx = lane; idx < R * D; idx += 64) {
          const int r = idx / D, d = idx - r * D;
          p.out[(static_cast<int64_t>(c.b) * p.H + u.hbase + r) * D + d] = 0.f;
          if (d == 0 && p.lse) p.lse[static_cast<int64_t>(c.b) * p.H + u.hbase + r] = kNegInf;
        }
      }
      return false;
    }
    u.t1 = min(u.t0 + split_size(p, c.split), L);
    const int64_t head0 = (PAGED ? 0 : static_cast<int64_t>(c.b) * p.max_seq_len * rs) +
                          static_cast<int64_t>(c.g) * (2 * D);
    u.kbase = static_cast<const char*>(p.k) + head0;
    u.vbase = static_cast<const char*>(p.v) + head0;
    return true;
  };
  // The next unit that holds tokens, starting from the claimed number in
  // `claimed_v` (lane 0); claims further units synchronously past empty
  // ones.  False when the units are exhausted.
  auto next_unit = [&](int claimed_v, Unit_& u) -> bool {
    int item = __builtin_amdgcn_readfirstlane(claimed_v);
    for (;;) {
      if (static_cast<uint32_t>(item) >= static_cast<uint32_t>(p.n_items)) return false;
      if (open_unit(item, u)) return true;
      item = __builtin_amdgcn_readfirstlane(claim());
    }
  };

  // paged: block ids of a unit, lane j of register c = block 64c + j of the
  // split; ids outside the pool become -1
  int blkv[PAGED ? kUnitBlkRegs : 1];
  auto load_blocks = [&](const Unit_& u) {
    if (!PAGED) return;
    const int nblk = (u.t1 - u.t0 + 15) >> 4;
    const int32_t* trow = p.table + static_cast<int64_t>(u.b) * p.max_blocks_per_seq + (u.t0 >> 4);
#pragma unroll
    for (int c = 0; c < kUnitBlkRegs; ++c) {
      const int i = c * 64 + lane;
      const int sb = i < nblk ? i : nblk - 1;
      const int blk = trow[sb];
      blkv[c] = (blk >= 0 && blk < p.num_blocks) ? blk : -1;
    }
  };
  // block ids (wave-uniform) of the two 16-token halves of tile kt
  auto tile_blocks = [&](int kt, int (&blk)[2]) {
    if (!PAGED) { blk[0] = blk[1] = 0; return; }
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const int i = 2 * kt + tb;
      int v = blkv[0];
#pragma unroll
      for (int c = 1; c < kUnitBlkRegs; ++c) v = (i >> 6) == c ? blkv[c] : v;
      blk[tb] = __builtin_amdgcn_readlane(v, i & 63);
    }
  };
  // Each 16-token half of a tile is read through two buffer descriptors
  // that start at the half's first token row and end at the last valid one:
  // tokens at or past the end of the split, and every token of an invalid
  // block, are out of range and read as zeros without touching memory.
  struct TileSrc { rsrc_t k[2], v[2]; };
  auto tile_src = [&](const Unit_& u, int tbase, const int (&blk)[2]) {
    TileSrc ts;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int lo = tbase + 16 * h;
      int rows = u.t1 - lo;
      rows = rows < 0 ? 0 : (rows > 16 ? 16 : rows);
      int64_t off;
      if (PAGED) {
        if (blk[h] < 0) rows = 0;
        off = static_cast<int64_t>(blk[h] < 0 ? 0 : blk[h]) * 16 * rs;
      } else {
        off = static_cast<int64_t>(lo) * rs;
      }
      const uint32_t bytes = static_cast<uint32_t>(rows) * static_cast<uint32_t>(rs);
      ts.k[h] = make_rsrc(u.kbase + off, bytes);
      ts.v[h] = make_rsrc(u.vbase + off, bytes);
    }
    return ts;
  };
  auto issue_k = [&](const TileSrc& ts, uint4 (&k)[2][KB]) {
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) k[tb][kb] = load16(ts.k[tb], koff + kb * 64);
  };
  // V rows, coalesced, HBM -> LDS: instruction jj covers tile rows
  // jj*RPI .. +RPI-1, i.e. rows (jj*RPI) % 16 + lane/LPR of half jj*RPI/16
  auto issue_v = [&](const TileSrc& ts, lds_char* buf) {
#pragma unroll
    for (int jj = 0; jj < NVL; ++jj) {
      const uint32_t off = vlane + static_cast<uint32_t>(((jj * RPI) % 16) * rs);
      copy16_to_lds(ts.v[(jj * RPI) / 16], buf + jj * G::BLOCK, off);
    }
  };
  // q operands: lane (n, grp) of block (nb, kb) holds dims kb*32 + grp*8
  // .. +7 of head nb*16 + n.  Unconditional vector loads from a valid head,
  // then a select (a load under a per-lane branch would serialise).
  float4 qraw[NB][KB][2];
  auto load_q = [&](const Unit_& u) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int h = nb * 16 + n;
      const float* src = p.q_rot + (static_cast<int64_t>(u.b) * p.H + u.hbase + (h < R ? h : 0)) * D + grp * 8;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        qraw[nb][kb][0] = *reinterpret_cast<const float4*>(src + kb * 32);
        qraw[nb][kb][1] = *reinterpret_cast<const float4*>(src + kb * 32 + 4);
      }
    }
  };
  bf16x8 qh[NB][KB], ql[NB][KB];
  // q * scale * log2(e) as bf16 hi + lo (heads >= n_rep get zeros)
  auto convert_q = [&]() {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const float qs = nb * 16 + n < R ? p.qscale : 0.f;
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
  };

  uint4 kr[2][KB];
  f32x4 acc[NB][CB];
  float m[NB], l[NB];

  // scores of the tile whose K rows are in `kr`
  auto scores = [&](f32x4 (&s)[NB][2]) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const bf16x8 a = __builtin_bit_cast(bf16x8, kr[h2][kb]);
          c = mfma(a, qh[nb][kb], c);
          c = mfma(a, ql[nb][kb], c);
        }
        s[nb][h2] = c;
      }
  };
  // online softmax of a tile's scores into P (hi, lo) and the running (m, l)
  auto softmax = [&](const Unit_& u, int tbase, f32x4 (&s)[NB][2], bool masked, bool ok0, bool ok1,
                     bf16x8 (&ph)[NB], bf16x8 (&pl)[NB]) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float sv[8];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int j = 0; j < 4; ++j) sv[h2 * 4 + j] = s[nb][h2][j];
      if (masked) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int t = tbase + 16 * h2 + 4 * grp + j;
            const bool ok = h2 == 0 ? ok0 : ok1;
            if (!(t < u.t1 && ok)) sv[h2 * 4 + j] = kNegInf;
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
  // zero the staged V rows that do not hold a valid token of the unit
  auto zero_masked_rows = [&](const Unit_& u, int tbase, int cur, bool ok0, bool ok1) {
    const uint32_t vt = lds_addr(vbuf[cur]);
#pragma unroll
    for (int jj = 0; jj < NVL; ++jj) {
      const int r = jj * RPI + lane / LPR;
      const bool ok = (jj * RPI) / 16 == 0 ? ok0 : ok1;
      if (!(tbase + r < u.t1 && ok)) lds_zero16(vt + jj * G::BLOCK + lane * 16);
    }
  };
  // O^T[d][h] += V^T[d][t] P^T[t][h]; A row = dim 16*cb + n, tokens 16*(j/4) + 4*grp + j%4
  auto pv = [&](int cur, const bf16x8 (&ph)[NB], const bf16x8 (&pl)[NB]) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const bf16x8 av = gather_v<D>(vrd[cur] + cb * 32);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        acc[nb][cb] = mfma(av, ph[nb], acc[nb][cb]);
        acc[nb][cb] = mfma(av, pl[nb], acc[nb][cb]);
      }
    }
  };
  // the unit's normalised output and log-sum-exp, from registers: lane
  // (n, grp) holds dims 16*cb + 4*grp .. +3 of head nb*16 + n
  auto write_unit = [&](const Unit_& u) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const float lt = l[nb] + __shfl_xor(l[nb], 16);
      const float lsum = lt + __shfl_xor(lt, 32);
      const int h = nb * 16 + n;
      if (h < R) {
        // every token of the unit masked (invalid blocks): empty softmax
        const bool any = lsum > 0.f;
        const float inv = any ? 1.f / lsum : 0.f;
        const float lse2 = any ? m[nb] + log2f(lsum) : kNegInf;
        const int64_t row = static_cast<int64_t>(u.b) * p.H + u.hbase + h;
        float* dst = p.direct ? p.out + row * D : p.part_o + (row * p.n_splits + u.split) * D;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const f32x4 a = acc[nb][cb];
          *reinterpret_cast<float4*>(dst + 16 * cb + 4 * grp) =
              make_float4(a[0] * inv, a[1] * inv, a[2] * inv, a[3] * inv);
        }
        if (grp == 0) {
          if (p.direct) {
            if (p.lse) p.lse[row] = lse2 * 0.69314718055994531f;
          } else {
            p.part_lse[row * p.n_splits + u.split] = lse2;
          }
        }
      }
    }
  };

  // ---------------------------------------------------------- the stream
  Unit_ cu;
  if (next_unit(claim(), cu)) {
    int cur = 0;                        // buffer holding the current tile's V rows
    int blk_cur[2];
    load_blocks(cu);
    load_q(cu);
    tile_blocks(0, blk_cur);
    {
      const TileSrc ts = tile_src(cu, cu.t0, blk_cur);
      issue_k(ts, kr);
      issue_v(ts, vbuf[0]);
    }
    for (;;) {
      const int next_v = claim();       // the unit after this one
      convert_q();
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        m[nb] = kNegInf; l[nb] = 0.f;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) acc[nb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      int base = cu.t0, kt = 0;
      // every tile but the last: the next tile of the unit is in flight
      while (base + TT < cu.t1) {
        int blk_next[2];
        tile_blocks(kt + 1, blk_next);
        const TileSrc ns = tile_src(cu, base + TT, blk_next);
        issue_v(ns, vbuf[cur ^ 1]);
        // keep the copies ahead of the score MFMAs, whose wait for `kr` may
        // then leave them outstanding
        __builtin_amdgcn_sched_barrier(0);
        const bool ok0 = !PAGED || blk_cur[0] >= 0;
        const bool ok1 = !PAGED || blk_cur[1] >= 0;
        const bool masked = !ok0 || !ok1;         // a full tile: only bad blocks mask
        f32x4 s[NB][2];
        scores(s);
        issue_k(ns, kr);                // K rows of the next tile, into the same registers
        bf16x8 ph[NB], pl[NB];
        softmax(cu, base, s, masked, ok0, ok1, ph, pl);
        // this tile's V copies have landed: only the next tile's loads (V
        // copies, then K rows) may still be outstanding
        vmem_wait<G::NLOADS>();
        if (masked) zero_masked_rows(cu, base, cur, ok0, ok1);
        pv(cur, ph, pl);
        blk_cur[0] = blk_next[0];
        blk_cur[1] = blk_next[1];
        base += TT;
        ++kt;
        cur ^= 1;
      }
      // the last tile: scores, then the next unit's first loads, then the rest
      const bool ok0 = !PAGED || blk_cur[0] >= 0;
      const bool ok1 = !PAGED || blk_cur[1] >= 0;
      const bool masked = base + TT > cu.t1 || !ok0 || !ok1;
      f32x4 s[NB][2];
      scores(s);
      // everything of this unit has landed (its last K rows were the last
      // loads issued): the next unit's loads may follow
      vmem_wait<0>();
      Unit_ nu;
      const bool more = next_unit(next_v, nu);
      if (more) {
        load_blocks(nu);
        load_q(nu);
        int blk0[2];
        tile_blocks(0, blk0);
        const TileSrc ts = tile_src(nu, nu.t0, blk0);
        issue_k(ts, kr);
        issue_v(ts, vbuf[cur ^ 1]);
        blk_cur[0] = blk0[0];
        blk_cur[1] = blk0[1];
      }
      bf16x8 ph[NB], pl[NB];
      softmax(cu, base, s, masked, ok0, ok1, ph, pl);
      if (masked) zero_masked_rows(cu, base, cur, ok0, ok1);
      pv(cur, ph, pl);
      write_unit(cu);
      if (!more) break;
      cu = nu;
      cur ^= 1;
    }
  }

  // the last wave to leave puts the counters back to zero for the next call
  if (lane == 0) {
    const uint32_t done = __hip_atomic_fetch_add(ctr + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (done == static_cast<uint32_t>(p.n_workers) - 1u) {
      __hip_atomic_exchange(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_exchange(ctr + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <int D, int NB, bool PAGED>
const void* kernel_fn() {
  return reinterpret_cast<const void*>(&decode_wave_kernel<D, NB, PAGED>);
}

template <int D, int NB>
hipError_t launch_nb(const DecodeParams& p, bool paged, int n_wg, hipStream_t s) {
  if (paged) decode_wave_kernel<D, NB, true><<<n_wg, 256, 0, s>>>(p);
  else decode_wave_kernel<D, NB, false><<<n_wg, 256, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_wave(const DecodeParams& p, bool paged, int n_wg, hipStream_t s) {
  if (p.chunk > kWaveMaxChunk || p.chunk % 16 != 0 || p.chunk2 > p.chunk || p.chunk2 < 16 ||
      p.chunk2 % 16 != 0 || p.n_big < 0 || p.n_big > p.n_splits || !p.counters || n_wg < 1 ||
      p.n_workers != n_wg * kMfmaWaves || p.R > 32)
    return hipErrorInvalidValue;
  if (p.D == 64) return p.R <= 16 ? launch_nb<64, 1>(p, paged, n_wg, s) : launch_nb<64, 2>(p, paged, n_wg, s);
  return p.R <= 16 ? launch_nb<128, 1>(p, paged, n_wg, s) : launch_nb<128, 2>(p, paged, n_wg, s);
}

int decode_wave_occupancy(int D, int R, bool paged) {
  const bool nb2 = R > 16;
  const void* fn;
  if (D == 64) {
    fn = nb2 ? (paged ? kernel_fn<64, 2, true>() : kernel_fn<64, 2, false>())
             : (paged ? kernel_fn<64, 1, true>() : kernel_fn<64, 1, false>());
  } else {
    fn = nb2 ? (paged ? kernel_fn<128, 2, true>() : kernel_fn<128, 2, false>())
             : (paged ? kernel_fn<128, 1, true>() : kernel_fn<128, 1, false>());
  }
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, 256, 0) != hipSuccess) return 0;
  return n;
}

}  // namespace kvd
