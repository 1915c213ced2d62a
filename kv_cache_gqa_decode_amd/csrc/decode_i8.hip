// Split-K decode attention over an INT8 KV cache on the matrix cores
// (D in {64, 128}, up to 32 query heads per KV head).
//
// The cache holds K and V as 8-bit codes n in [-127, 127] with one fp32
// scale per KV head for each ("Transformer推理核心：KV Cache、GQA与RoPE原理与工程实践"
// §4.3: INT8 K/V with per-head quantisation parameters), so an element's
// value is scale[g] * n and the result is softmax(q K^T * scale) V over those
// values, as for the other dtypes (§2.1, §4.2 of the same page).  Half the
// bytes of bf16 per token: the same HBM roof streams twice the tokens.
//
// Layout: tokens grouped by 16, each group holding per KV head its 16 K rows
// ([G][16][D]) and its V block transposed ([G][D][16]): a tile's K and V of
// one head are 2 KB runs (at D = 128) instead of 128-byte rows 1 KB apart,
// which streamed 5-12% faster in measurement, and one 16-byte V^T load gives
// a lane sixteen tokens of one dimension -- the operand layout of the P V
// product, with no transpose on the way.
//
// Per wave and 64-token tile (four 16-token groups):
//   scores  v_mfma_i32_16x16x64_i8 on the codes themselves.  A = K rows
//           (16 bytes of one token per lane, straight from HBM), B = q as
//           three int8 limbs: q * (127 / max|q_h|) = a1 + a2/128 + a3/128^2
//           up to 2^-15, each limb a separate exact int32 product.  The
//           scores are sum_l S_l * 128^(1-l) * scale * k_scale * max|q_h|/127,
//           relative accuracy ~2^-22 of the row -- the fp32 q enters exactly
//           enough while K stays exact.  Rows of the score tile are permuted
//           so that lane group c ends up holding the sixteen tokens of group
//           c of the tile: half hb, row 4c + j is token 16c + 4hb + j.
//   softmax running max / sum per head as in the bf16 kernel (lazy rescale by
//           2^8 slack); probabilities are taken as 2^6 p so that their
//           fp16 split stays in the normal range (the factor cancels in the
//           normalisation; the stored max is lowered by 6 to match).
//   P V     O^T[d][h] += sum_t V^T[d][t] P^T[t][h] with
//           v_mfma_f32_16x16x32_f16: A = the V^T row of the lane's token
//           group turned into fp16 exactly (c XOR 0x80 under the exponent
//           byte 0x64 is the half 1152 + c, minus 1152), B = P split into
//           fp16 hi + lo.  The final output is multiplied by v_scale.
//
// Pipeline: both operands are double-buffered and tile i+1 is requested
// before tile i is computed -- its K rows into the second K register set,
// its V^T blocks HBM -> LDS with buffer_load ... lds (no registers; each
// copy instruction lands 1 KiB of one group's V^T block) into the wave's
// second LDS buffer -- so a wave keeps up to two tiles (32 KB at D = 128)
// in flight and each tile's loads have a whole tile of compute to arrive.
// One wait per tile ("at most one tile of loads outstanding") covers both.
// The V^T reads from LDS are inline assembly for the reason given with
// read_vt_tr in mfma_tile.h (the compiler would otherwise wait for every
// outstanding copy first).  K rows past the end of the split are read from
// the last group that holds a token (always inside the cache); V^T blocks
// past it, or of an invalid block, are read out of range (zeros, no memory
// traffic).  Masked tokens get probability 0, and codes are finite, so they
// contribute exactly zero.
#include "i8_codes.h"

namespace kvd {
namespace {

using namespace mt;

typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kTT = kI8TileTokens;     // tokens per wave-tile
constexpr int kLimbs = 3;
constexpr float kPBias = 6.f;          // probabilities carried as 2^6 p
constexpr int kBlkRegsI8 = (kMaxChunk / 16 / kMfmaWaves + 63) / 64;

__device__ __forceinline__ i32x4 mfma_i8(i32x4 a, i32x4 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}
// fp16 hi + lo of two floats (hi truncated, lo the exact remainder truncated:
// hi + lo within 2^-21 of x).
__device__ __forceinline__ void split_f16(float a, float b, uint32_t& hi, uint32_t& lo) {
  const auto h = __builtin_amdgcn_cvt_pkrtz(a, b);
  const auto l = __builtin_amdgcn_cvt_pkrtz(a - static_cast<float>(h[0]),
                                            b - static_cast<float>(h[1]));
  hi = __builtin_bit_cast(uint32_t, h);
  lo = __builtin_bit_cast(uint32_t, l);
}

__device__ __forceinline__ uint32_t pack4(int a, int b, int c, int d) {
  return (static_cast<uint32_t>(a) & 255u) | ((static_cast<uint32_t>(b) & 255u) << 8) |
         ((static_cast<uint32_t>(c) & 255u) << 16) | (static_cast<uint32_t>(d) << 24);
}

// Sixteen bytes of each of this lane's CB V^T rows from LDS (row cb at
// addr + 256 cb), waiting for its own reads.  Inline assembly: see read_vt_tr.
template <int CB>
__device__ __forceinline__ void read_vt(uint32_t addr, u32x4 (&v)[CB]);
template <>
__device__ __forceinline__ void read_vt<8>(uint32_t addr, u32x4 (&v)[8]) {
  asm volatile(
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %8 offset:256\n\t"
      "ds_read_b128 %2, %8 offset:512\n\t"
      "ds_read_b128 %3, %8 offset:768\n\t"
      "ds_read_b128 %4, %8 offset:1024\n\t"
      "ds_read_b128 %5, %8 offset:1280\n\t"
      "ds_read_b128 %6, %8 offset:1536\n\t"
      "ds_read_b128 %7, %8 offset:1792\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]),
        "=&v"(v[6]), "=&v"(v[7])
      : "v"(addr));
}
template <>
__device__ __forceinline__ void read_vt<4>(uint32_t addr, u32x4 (&v)[4]) {
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %4 offset:256\n\t"
      "ds_read_b128 %2, %4 offset:512\n\t"
      "ds_read_b128 %3, %4 offset:768\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
      : "v"(addr));
}

// LDS of a workgroup: two staged V^T tiles (64 D bytes each) per wave,
// reused for the merge of the waves
template <int D>
constexpr int smem_bytes_i8() {
  constexpr int stage = kMfmaWaves * 2 * 64 * D;
  constexpr int merge = merge_bytes<D>();
  return stage > merge ? stage : merge;
}

// One (sequence b, KV head g, split) unit computed by the whole workgroup:
// query rows rb .. rb + 16 NB - 1 of the KV head (rb > 0 when the rows are
// split over row groups).
typedef __attribute__((address_space(3))) double lds_f64;

// FUSED (the decode step in one launch, one new token, NB = 1, no row
// groups): q is rotated here from the raw q, and the workgroup of the
// sequence's last split quantises and appends the token's k and v first.
template <int D, int NB, bool PAGED, bool FUSED = false>
__device__ __forceinline__ void run_split_i8(const DecodeParams& p, char* smem, int b, int g,
                                             int split, int rb) {
  constexpr int KB = D / 64;          // 64-dim blocks of the score contraction
  constexpr int CB = D / 16;          // 16-dim blocks of the output
  constexpr int kWaves = kMfmaWaves;
  constexpr int kGroupBytes = 16 * D; // V^T block of one group and head
  constexpr int kTileBytes = 4 * kGroupBytes;
  constexpr int NK = 4 * KB;          // K loads per tile
  constexpr int NV = kTileBytes / 1024;   // V^T copy instructions per tile
  static_assert(NB >= 1 && NB <= 2 && (D == 64 || D == 128), "tile shape");
  static_assert(!FUSED || NB == 1, "the fused step takes up to 16 query rows");
  const int R = p.R;
  const int RT = R * p.T;             // tile columns: the query rows of this KV head
  const int raw_len = scalar_load_i32(p.seq_lens + b);   // FUSED: the new token's position
  const int L = attended_len(p, len_of(p, raw_len));
  const int t0 = split_start(p, split);
  if (t0 >= L) {
    if (p.direct && split == 0) {     // empty sequence: out = 0, lse = -inf
      const int nr = min(16 * NB, RT - rb);
      for (int idx = threadIdx.x; idx < nr * D; idx += 256) {
        const int r = idx / D, d = idx - r * D;
        const int64_t row = query_row(p, b, g, rb + r);
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
    const int c = rb + nb * 16 + (threadIdx.x & 15);
    cbound[nb] = c < RT ? win + c / R : L;
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, grp = lane >> 4;
  // bytes per 16-token group (all heads), and the start of head g's K rows
  // and V^T block in group 0 (of sequence b when contiguous)
  const int64_t gs = static_cast<int64_t>(p.G) * D * 16;
  const int8_t* kbase = static_cast<const int8_t*>(p.k) + static_cast<int64_t>(g) * D * 16;
  const int8_t* vbase = static_cast<const int8_t*>(p.v) + static_cast<int64_t>(g) * D * 16;
  if (!PAGED) {
    kbase += static_cast<int64_t>(b) * (p.max_seq_len >> 4) * gs;
    vbase += static_cast<int64_t>(b) * (p.max_seq_len >> 4) * gs;
  }

  // q rows, requested first: lane (n, grp) of block (nb, kb) holds dims
  // kb*64 + grp*16 .. +15 of head nb*16 + n.  With two column blocks the
  // rows are loaded once per workgroup and staged in LDS (QStage).
  float4 qraw[NB][KB][4];
  QStage<D> qst;
  // FUSED: the raw q (bf16), rotated once the factors are in LDS
  uint4 qin[FUSED ? 2 * KB : 1];
  if constexpr (NB == 2) {
    qst.load(p, b, g, RT, wave, lane);
  } else if constexpr (FUSED) {
    const uint16_t* src = static_cast<const uint16_t*>(p.q_in) +
                          (static_cast<int64_t>(b) * p.H + g * R + (n < RT ? n : 0)) * D + grp * 16;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      qin[2 * kb] = *reinterpret_cast<const uint4*>(src + kb * 64);
      qin[2 * kb + 1] = *reinterpret_cast<const uint4*>(src + kb * 64 + 8);
    }
  } else {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int h = rb + nb * 16 + n;
      const float* src = p.q_rot + query_row(p, b, g, h < RT ? h : 0) * D + grp * 16;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          qraw[nb][kb][j] = *reinterpret_cast<const float4*>(src + kb * 64 + 4 * j);
    }
  }

  // paged: the ids of the blocks this wave visits, lane j of register c =
  // the wave's (64c + j)-th block = split block 16*(i/4) + 4*wave + i%4 with
  // i = 64c + j (group i%4 of the wave's tile i/4); ids outside the pool
  // become -1
  int blkv[PAGED ? kBlkRegsI8 : 1];
  const int last_grp = (t1 - 1) >> 4;         // last group holding a token of the split
  if (PAGED) {
    const int nblk = last_grp - (t0 >> 4) + 1;
#pragma unroll
    for (int c = 0; c < kBlkRegsI8; ++c) {
      const int i = c * 64 + lane;
      int sb = 16 * (i >> 2) + 4 * wave + (i & 3);
      sb = sb < nblk ? sb : nblk - 1;
      blkv[c] = paged_group(p, b, (t0 >> 4) + sb);
    }
  }

  // K rows of tile kt (first token tbase) into `k`: the lane reads rows of
  // group n/4 of the tile (groups past the split's last one are replaced by
  // it: in bounds, and masked); `vok` = the lane's own group grp is a valid
  // block (paged), i.e. its tokens may be attended
  auto issue_k = [&](int tbase, int kt, i32x4 (&k)[4][KB], bool& vok) {
    int64_t kgo;
    if (PAGED) {
      int src = blkv[0];
#pragma unroll
      for (int c = 1; c < kBlkRegsI8; ++c) src = (kt >> 4) == c ? blkv[c] : src;
      const int ik = __shfl(src, (4 * kt + (n >> 2)) & 63);
      const int iv = __shfl(src, (4 * kt + grp) & 63);
      kgo = ik < 0 ? 0 : ik;
      vok = iv >= 0;
    } else {
      const int gk = (tbase >> 4) + (n >> 2);
      kgo = gk < last_grp ? gk : last_grp;
      vok = true;
    }
    const int8_t* ka = kbase + kgo * gs + (n & 3) * D + grp * 16;
#pragma unroll
    for (int hb = 0; hb < 4; ++hb)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        k[hb][kb] = *reinterpret_cast<const i32x4*>(ka + hb * 4 * D + kb * 64);
  };
  // V^T blocks of the tile's four groups, HBM -> LDS buffer `buf` (group x
  // at x * kGroupBytes); groups past the split or invalid blocks read nothing
  auto issue_v = [&](int tbase, int kt, lds_char* buf) {
    int src = 0;
    if (PAGED) {
      src = blkv[0];
#pragma unroll
      for (int c = 1; c < kBlkRegsI8; ++c) src = (kt >> 4) == c ? blkv[c] : src;
    }
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int g16 = (tbase >> 4) + x;
      bool ok = g16 <= last_grp;
      const int8_t* blk = vbase;
      if (PAGED) {
        const int id = __builtin_amdgcn_readlane(src, (4 * kt + x) & 63);
        ok = ok && id >= 0;
        if (ok) blk = vbase + static_cast<int64_t>(id) * gs;
      } else if (ok) {
        blk = vbase + static_cast<int64_t>(g16) * gs;
      }
      const rsrc_t r = make_rsrc(reinterpret_cast<const char*>(blk), ok ? kGroupBytes : 0u);
#pragma unroll
      for (int h = 0; h < kGroupBytes / 1024; ++h)
        copy16_to_lds(r, buf + x * kGroupBytes + h * 1024, static_cast<uint32_t>(lane * 16 + h * 1024));
    }
  };

  lds_char* const stage = (lds_char*)(smem);
  lds_char* const vb0 = stage + (2 * wave) * kTileBytes;
  lds_char* const vb1 = stage + (2 * wave + 1) * kTileBytes;
  // this lane's V^T row (dim 16cb + n of group grp) in each buffer
  const uint32_t vrd0 = lds_addr(vb0) + grp * kGroupBytes + n * 16;
  const uint32_t vrd1 = lds_addr(vb1) + grp * kGroupBytes + n * 16;

  i32x4 kr0[4][KB], kr1[4][KB];
  int base = t0 + wave * kTT;
  bool vok0 = true, vok1 = true;
  // With two column blocks the first tile is requested on every path (a
  // wave without tiles reads its split's last group of K, in bounds, and
  // copies nothing: empty descriptors), so the compiler's wait for the q
  // rows it stages stays partial instead of also waiting for this tile.
  // With one block the request stays under the branch: issuing it on every
  // path measured 2-3% slower on a 128K GQA sequence (same box, A/B).
  // FUSED: the workgroup of the last split appends the new token (wave-
  // uniform), and must not request its first tile before that
  const bool appender = FUSED && split == split_count(p, L) - 1;
  if (!appender && (NB == 2 || base < t1)) {
    issue_v(base, 0, vb0);
    issue_k(base, 0, kr0, vok0);
  }
  if constexpr (FUSED) {
    // RoPE factors of the new token's position, fp64 as the append kernel
    // computes them, into wave 0's second V buffer (free until its second
    // tile)
    const int P = raw_len;
    lds_f64* const fcos = reinterpret_cast<lds_f64*>(stage + kTileBytes);
    lds_f64* const fsin = fcos + D / 2;
    if (wave == 0 && lane < D / 2) {
      const double theta = pow(p.rope_base, -2.0 * lane / D);
      double sv, cv;
      sincos(static_cast<double>(P) * theta, &sv, &cv);
      fcos[lane] = cv;
      fsin[lane] = sv;
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const bool inter = p.rope_style != KVD_ROPE_HALF;
    if (appender) {
      // the codes of the rotated k_new and of v_new in the token's slot of
      // its 16-token group (skipped outside the cache); the stores land
      // before any wave requests a tile, and the tile that holds P reads
      // them
      if (P >= 0 && P < p.max_seq_len) {
        const int64_t grp16 = PAGED ? paged_group(p, b, P >> 4)
                                    : static_cast<int64_t>(b) * (p.max_seq_len >> 4) + (P >> 4);
        if (grp16 >= 0) {
          const int64_t src = (static_cast<int64_t>(b) * p.G + g) * D;
          const uint16_t* kn = static_cast<const uint16_t*>(p.k_new) + src;
          int8_t* kc = static_cast<int8_t*>(const_cast<void*>(p.k)) +
                       ((grp16 * p.G + g) * 16 + (P & 15)) * D;
          const int i = threadIdx.x;
          if (i < D / 2) {
            const int ia = inter ? 2 * i : i, ib = inter ? 2 * i + 1 : i + D / 2;
            const double a = bf16_to_float(kn[ia]), c = bf16_to_float(kn[ib]);
            const double cf = fcos[i], sf = fsin[i];
            const float ks = p.k_scale[g];
            kc[ia] = quantize_i8(a * cf - c * sf, ks);
            kc[ib] = quantize_i8(a * sf + c * cf, ks);
          } else if (i < D / 2 + D) {
            const int d = i - D / 2;
            int8_t* vc = static_cast<int8_t*>(const_cast<void*>(p.v));
            vc[((grp16 * p.G + g) * D + d) * 16 + (P & 15)] =
                quantize_i8(bf16_to_float(static_cast<const uint16_t*>(p.v_new)[src + d]),
                            p.v_scale[g]);
          }
        }
      }
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
      if (base < t1) {
        issue_v(base, 0, vb0);
        issue_k(base, 0, kr0, vok0);
      }
    }
    // rotate this lane's 16 dims per 64-dim block, fp64, rounded once to
    // fp32 as q_rot: interleaved pairs sit in the lane's dims; half pairs
    // in blocks kb and kb + KB/2 (D = 128) or in the lane 32 apart (D = 64)
    float qv[KB][16];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const uint32_t w[8] = {qin[2 * kb].x, qin[2 * kb].y, qin[2 * kb].z, qin[2 * kb].w,
                             qin[2 * kb + 1].x, qin[2 * kb + 1].y, qin[2 * kb + 1].z,
                             qin[2 * kb + 1].w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        qv[kb][2 * j] = bf16lo(w[j]);
        qv[kb][2 * j + 1] = bf16hi(w[j]);
      }
    }
    if (inter) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int f = kb * 32 + grp * 8 + j;
          const double a = qv[kb][2 * j], c = qv[kb][2 * j + 1];
          const double cf = fcos[f], sf = fsin[f];
          qv[kb][2 * j] = static_cast<float>(a * cf - c * sf);
          qv[kb][2 * j + 1] = static_cast<float>(a * sf + c * cf);
        }
    } else if constexpr (KB == 2) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int f = grp * 16 + e;
        const double a = qv[0][e], c = qv[1][e];
        const double cf = fcos[f], sf = fsin[f];
        qv[0][e] = static_cast<float>(a * cf - c * sf);
        qv[1][e] = static_cast<float>(a * sf + c * cf);
      }
    } else {
      // D = 64: dims grp*16 + e; the partner of dim d < 32 is d + 32, held
      // by the lane with grp + 2 (lane ^ 32)
      const bool low = grp < 2;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float other = __shfl_xor(qv[0][e], 32);
        const int f = (grp & 1) * 16 + e;
        const double own = qv[0][e], par = other;
        const double cf = fcos[f], sf = fsin[f];
        qv[0][e] = low ? static_cast<float>(own * cf - par * sf)
                       : static_cast<float>(par * sf + own * cf);
      }
    }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        qraw[0][kb][j] = make_float4(qv[kb][4 * j], qv[kb][4 * j + 1], qv[kb][4 * j + 2],
                                     qv[kb][4 * j + 3]);
    // q_rot for the caller, written once per (sequence, KV head)
    if (p.q_rot_out && split == 0 && n < RT) {
      float* dst = p.q_rot_out + (static_cast<int64_t>(b) * p.H + g * R + n) * D + grp * 16;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j) *reinterpret_cast<float4*>(dst + kb * 64 + 4 * j) = qraw[0][kb][j];
    }
    // every wave has read the factors before wave 0 copies its second tile
    // over them
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }

  if constexpr (NB == 2) {
    const uint32_t st = lds_addr(stage);
    qst.publish(st, kTileBytes, wave, lane);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int h = nb * 16 + n;
      const uint32_t a = QStage<D>::row_addr(st, kTileBytes, h < RT ? h : 0) + 64 * grp;
      static_for<KB>([&](auto kbc) {
        constexpr int kb = decltype(kbc)::value;
        read_b128x2<256 * kb>(a, qraw[nb][kb][0], qraw[nb][kb][1]);
        read_b128x2<256 * kb + 32>(a, qraw[nb][kb][2], qraw[nb][kb][3]);
      });
    }
    __builtin_amdgcn_s_barrier();      // every wave's q read before the rows are reused
  }

  // q as three int8 limbs per head, and the per-head factors that turn the
  // limbs' int32 products back into scores (log2 units)
  i32x4 ql[kLimbs][NB][KB];
  float mul[kLimbs][NB];
  const float kscale = p.k_scale[g];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const bool real = rb + nb * 16 + n < RT;
    float amax = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 x = qraw[nb][kb][j];
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(x.x), fabsf(x.y)), fmaxf(fabsf(x.z), fabsf(x.w))));
      }
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    const float c = real && amax > 0.f ? 127.f / amax : 0.f;
    const float m1 = real ? p.qscale * kscale * (amax / 127.f) : 0.f;
    mul[0][nb] = m1;
    mul[1][nb] = m1 * (1.f / 128.f);
    mul[2][nb] = m1 * (1.f / 16384.f);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      int a[kLimbs][16];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 x = qraw[nb][kb][j];
        const float xv[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float y = xv[e] * c;
          const float a1 = __builtin_rintf(y);
          y = (y - a1) * 128.f;
          const float a2 = __builtin_rintf(y);
          y = (y - a2) * 128.f;
          const float a3 = __builtin_rintf(y);
          a[0][4 * j + e] = static_cast<int>(a1);
          a[1][4 * j + e] = static_cast<int>(a2);
          a[2][4 * j + e] = static_cast<int>(a3);
        }
      }
#pragma unroll
      for (int l = 0; l < kLimbs; ++l)
        ql[l][nb][kb] = i32x4{static_cast<int>(pack4(a[l][0], a[l][1], a[l][2], a[l][3])),
                              static_cast<int>(pack4(a[l][4], a[l][5], a[l][6], a[l][7])),
                              static_cast<int>(pack4(a[l][8], a[l][9], a[l][10], a[l][11])),
                              static_cast<int>(pack4(a[l][12], a[l][13], a[l][14], a[l][15]))};
    }
  }

  f32x4 acc[NB][CB];
  float m[NB], lsum[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    m[nb] = kNegInf; lsum[nb] = 0.f;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[nb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // One tile (the wave's kt-th, first token tbase): K rows in `kc`, V^T in
  // the LDS buffer read at `vrc`, `vokc` its lane-group validity.  `more` (a
  // constant at each call) says whether there is a next tile, whose loads
  // then go out first, into `kn` and the other LDS buffer `vbn`.
  auto compute = [&](int kt, int tbase, i32x4 (&kc)[4][KB], i32x4 (&kn)[4][KB], lds_char* vbn,
                     uint32_t vrc, bool vokc, bool& vokn, const bool more) {
    if (more) {
      issue_v(tbase + kWaves * kTT, kt + 1, vbn);
      issue_k(tbase + kWaves * kTT, kt + 1, kn, vokn);
      // every load of the next tile goes out before anything of this one is
      // computed (the compiler would hoist the score MFMAs above the later
      // loads and then wait for this tile's K rows early)
      __builtin_amdgcn_sched_barrier(0);
      vmem_wait<NK + NV>();            // this tile's K rows and V^T blocks have landed
    } else {
      vmem_wait<0>();
    }
    const bool full = tbase + kTT <= t1;
    const bool masked = !full || (PAGED && !__all(vokc)) || tbase + kTT > win;   // wave-uniform
    // int32 score products of the three limbs, half hb = token rows
    // 16c + 4hb + j of the tile's groups c
    i32x4 S[kLimbs][NB][4];
#pragma unroll
    for (int l = 0; l < kLimbs; ++l)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) {
          i32x4 c = {0, 0, 0, 0};
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) c = mfma_i8(kc[hb][kb], ql[l][nb][kb], c);
          S[l][nb][hb] = c;
        }

    f16x8 ph[NB][2], pl[NB][2];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float sv[16];
#pragma unroll
      for (int hb = 0; hb < 4; ++hb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float s1 = static_cast<float>(S[0][nb][hb][j]);
          const float s2 = static_cast<float>(S[1][nb][hb][j]);
          const float s3 = static_cast<float>(S[2][nb][hb][j]);
          sv[hb * 4 + j] = fmaf(s3, mul[2][nb], fmaf(s2, mul[1][nb], s1 * mul[0][nb]));
        }
      if (masked) {
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int t = tbase + 16 * grp + 4 * hb + j;
            if (!(t < t1 && vokc && t < cbound[nb])) sv[hb * 4 + j] = kNegInf;
          }
      }
      float mt = sv[0];
#pragma unroll
      for (int j = 1; j < 16; ++j) mt = fmaxf(mt, sv[j]);
      mt = fmaxf(mt, __shfl_xor(mt, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      if (__builtin_expect(__any(mt > m[nb] + kRescaleSlack), 0)) {   // a running max moves
        const float mn = fmaxf(m[nb], mt);
        const float alpha = mn == kNegInf ? 1.f : __builtin_amdgcn_exp2f(m[nb] - mn);
        lsum[nb] *= alpha;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) acc[nb][cb] *= alpha;
        m[nb] = mn;
      }
      const float ref = (m[nb] == kNegInf ? 0.f : m[nb]) - kPBias;
      float pv[16];
      float ps = 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        pv[j] = __builtin_amdgcn_exp2f(sv[j] - ref);
        ps += pv[j];
      }
      lsum[nb] += ps;
      // B operand of k-block kk: tokens 8kk .. 8kk+7 of the lane's group =
      // halves 2kk (rows j) and 2kk+1
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        uint32_t h[4], lo[4];
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2)
          split_f16(pv[8 * kk + 2 * q2], pv[8 * kk + 2 * q2 + 1], h[q2], lo[q2]);
        ph[nb][kk] = __builtin_bit_cast(f16x8, u32x4{h[0], h[1], h[2], h[3]});
        pl[nb][kk] = __builtin_bit_cast(f16x8, u32x4{lo[0], lo[1], lo[2], lo[3]});
      }
    }

    // O^T[d][h] += V^T[d][t] P^T[t][h]; A row = dim 16cb + n, tokens of group grp
    u32x4 vt[CB];
    read_vt<CB>(vrc, vt);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const f16x8 a0 = codes_to_f16(vt[cb][0], vt[cb][1]);
      const f16x8 a1 = codes_to_f16(vt[cb][2], vt[cb][3]);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        acc[nb][cb] = mfma_f16(a0, ph[nb][0], acc[nb][cb]);
        acc[nb][cb] = mfma_f16(a0, pl[nb][0], acc[nb][cb]);
        acc[nb][cb] = mfma_f16(a1, ph[nb][1], acc[nb][cb]);
        acc[nb][cb] = mfma_f16(a1, pl[nb][1], acc[nb][cb]);
      }
    }
  };

  // K register sets and V buffers alternate; the wave's last tile issues no
  // loads
  if (base < t1) {
    int kt = 0;
    for (;;) {
      if (base + kWaves * kTT >= t1) { compute(kt, base, kr0, kr1, vb1, vrd0, vok0, vok1, false); break; }
      compute(kt, base, kr0, kr1, vb1, vrd0, vok0, vok1, true);
      base += kWaves * kTT;
      ++kt;
      if (base + kWaves * kTT >= t1) { compute(kt, base, kr1, kr0, vb0, vrd1, vok1, vok0, false); break; }
      compute(kt, base, kr1, kr0, vb0, vrd1, vok1, vok0, true);
      base += kWaves * kTT;
      ++kt;
    }
  }
  // a wave without tiles still has its first tile's loads outstanding (the
  // empty copies write zeros into its staging buffer, which the merge reuses)
  vmem_wait<0>();

  // per-wave sums: the four lane groups of a head hold partial sums under one max
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    lsum[nb] += __shfl_xor(lsum[nb], 16);
    lsum[nb] += __shfl_xor(lsum[nb], 32);
  }

  // merge the waves through LDS, 16 rows at a time; each wave's (max, sum,
  // O) is stated against max - kPBias, the scale its probabilities carry,
  // and O is in V codes (times v_scale)
  const float vscale = p.v_scale[g];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int nh = min(16, RT - rb - nb * 16);
    if (nh <= 0) break;
    merge_waves<D>(p, smem, b, g, split, rb + nb * 16, nh, acc[nb],
                   m[nb] == kNegInf ? kNegInf : m[nb] - kPBias, lsum[nb], vscale);
  }
}

// Up to 16 query heads per KV head: two workgroups per CU fit only if the
// registers stay within 256 per lane, which the compiler is told to aim for.
template <int D, bool PAGED, bool FUSED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void decode_i8_kernel(DecodeParams p) {
  __shared__ __align__(16) char smem[smem_bytes_i8<D>()];
  Unit u;
  if (!unit_at(p, u)) return;
  // with row groups the unit's head index is (KV head, row group)
  const int rg = p.row_groups > 1 ? p.row_groups : 1;
  run_split_i8<D, 1, PAGED, FUSED>(p, smem, u.b, u.g / rg, u.split, 16 * (u.g % rg));
}
// 17 to 32 query rows per KV head (two column blocks): at D = 128 the q
// limbs, scores and accumulators of the second block do not fit beside the
// double-buffered K registers within 256 per lane (held there, the compiler
// spills), so one workgroup per CU
template <int D, bool PAGED>
__global__ __launch_bounds__(256) void decode_i8_kernel_wide(DecodeParams p) {
  __shared__ __align__(16) char smem[smem_bytes_i8<D>()];
  Unit u;
  if (!unit_at(p, u)) return;
  run_split_i8<D, 2, PAGED>(p, smem, u.b, u.g, u.split, 0);
}

template <int D, int NB>
hipError_t launch_nb(const DecodeParams& p, bool paged, const Launch& l) {
  void (*k)(DecodeParams) =
      NB == 1 ? (p.len_bias ? (paged ? decode_i8_kernel<D, true, true> : decode_i8_kernel<D, false, true>)
                            : (paged ? decode_i8_kernel<D, true, false> : decode_i8_kernel<D, false, false>))
              : (paged ? decode_i8_kernel_wide<D, true> : decode_i8_kernel_wide<D, false>);
  return launch_kernel(k, split_grid(p), dim3(256), l, p);
}

// Up to 16 rows per workgroup: the one-block kernel (with row groups, each
// takes 16 of the head's rows); 17 to 32 in one workgroup: the wide kernel.
template <int D>
hipError_t launch_d(const DecodeParams& p, bool paged, const Launch& l) {
  return p.R * p.T <= 16 || p.row_groups > 1 ? launch_nb<D, 1>(p, paged, l)
                                             : launch_nb<D, 2>(p, paged, l);
}

}  // namespace

hipError_t launch_decode_i8(const DecodeParams& p, bool paged, const Launch& l) {
  if (p.chunk > kMaxChunk || p.chunk % 16 != 0 || p.chunk2 > p.chunk || p.chunk2 < 16 ||
      p.chunk2 % 16 != 0 || p.n_big < 0 || p.n_big > p.n_splits || p.T < 1 || p.R * p.T > 32 ||
      !p.k_scale || !p.v_scale || (!paged && p.max_seq_len % 16 != 0))
    return hipErrorInvalidValue;
  // row groups of 16 rows must cover the head's rows exactly
  if (p.row_groups > 1 && (p.row_groups != 2 || p.R * p.T <= 16)) return hipErrorInvalidValue;
  // the fused step: one new token, up to 16 query rows in one workgroup
  if (p.len_bias && (p.len_bias != 1 || p.T != 1 || p.R > 16 || p.row_groups > 1 || !p.q_in ||
                     !p.k_new || !p.v_new))
    return hipErrorInvalidValue;
  return p.D == 64 ? launch_d<64>(p, paged, l) : launch_d<128>(p, paged, l);
}

}  // namespace kvd
