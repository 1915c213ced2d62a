// Causal prefill attention over an INT8 cache on the fp16 matrix cores.
//
// "Transformer推理核心：KV Cache、GQA与RoPE原理与工程实践" §4.3: K and V held as
// 8-bit codes with per-head scales (value = scale[g] * code); §4.2: the tiled
// attention with an online softmax across key blocks; §5.1 b.v: the causal
// mask.  Query t of sequence b attends the tokens j < L_b - T + 1 + t, as in
// the bf16 prefill kernel, whose organisation this kernel keeps: a
// workgroup owns 128 query rows of one KV head (each wave 32), walks the
// 32-token key tiles below their bounds, and computes S^T = K Q^T and
// O^T = V^T P^T so that each row's softmax lives in one lane column.
//
// What differs is the cache: the INT8 layout groups tokens by 16, each group
// holding per KV head its 16 K rows [16][D] and its V block transposed
// [D][16].  Per tile:
//   * the two groups' K rows and V^T blocks (half the bytes of a bf16 tile)
//     are copied HBM -> LDS by the four waves;
//   * after a barrier the workgroup converts them once, cooperatively, into
//     an fp16 tile: every code is exact in fp16 (codes_to_f16), K rows go
//     to the bf16 kernel's swizzled row layout, and the V^T rows keep their
//     transposed form with the tokens reordered so that the 8 tokens a lane
//     feeds to the P V matrix op are contiguous -- no transposing read;
//   * after a second barrier the next tile's copies go out and the waves
//     compute on the fp16 tile.
// Converting once per workgroup costs each wave a quarter of a tile's codes;
// converting operands as each wave reads them would cost all four waves the
// whole tile.
//
// Arithmetic: q * scale * log2 e and the probabilities enter the matrix
// cores rounded once to fp16 (finer than the bf16 prefill's rounding),
// accumulation is fp32.  The raw scores q . code are multiplied by k_scale[g]
// before the softmax, the output by v_scale[g]; one fp32 running sum of the
// probabilities normalises the output and gives the log-sum-exp.  Key splits
// and dispatch orders are those of the bf16 prefill kernel.
#include "i8_codes.h"

namespace kvd {
namespace {

using namespace mt;

constexpr int kWaves = 4;
constexpr int kCols = 32;                        // query rows per wave
constexpr int kRows = kWaves * kCols;            // query rows per workgroup
constexpr int kTT = 32;                          // key tokens per tile
constexpr float kRescaleBound = 256.f;           // 2^kRescaleSlack
static_assert(kRescaleSlack == 8.f, "kRescaleBound is 2^kRescaleSlack");
static_assert(kRows == kPrefillRows && kTT == kPrefillTile, "the host plans with these");

template <int D>
struct I8PfGeo {
  static constexpr int KB = D / 32;              // 32-dim blocks of the score contraction
  static constexpr int CB = D / 16;              // 16-dim blocks of the output
  static constexpr int NDC = D / 8;              // 8-dim (16-byte fp16) chunks of a K row
  static constexpr int kGroup = 16 * D;          // bytes of one head's group: K rows or V^T
  static constexpr int kStage = 4 * kGroup;      // staged codes: K of 2 groups, then V^T
  static constexpr int NCI = kStage / 1024;      // copy instructions per tile
  // fp16 K row: 2D bytes and 32 of padding, so that row t starts 2t slots
  // (of 16 bytes) further round the banks than row 0
  static constexpr int kKRow = 2 * D + 32;
  static constexpr int kKBytes = kTT * kKRow;    // fp16 K tile
  // fp16 V^T row: 32 tokens and 32 bytes of padding.  96 bytes = 6 slots of
  // 16: the eight rows n = 0..7 a 16-byte read pass takes (lanes 0-7 and
  // 16-23, see swz) start on even slots 6 n mod 16, and the two lane groups
  // of the pass read slots 0 and 1 of them: all 16 slots, no conflict.
  static constexpr int kVRow = kTT * 2 + 32;
  static constexpr int kVBytes = D * kVRow;
  static constexpr int kLds = kStage + kKBytes + kVBytes;
  static_assert(NCI % kWaves == 0, "copies split over the waves");
  // K rows: chunk dc of row t at kat(t, dc), in plain order within its
  // padded row.  The score matrix op takes K row 16 h2 + n in lane n (tokens
  // in their own order, unlike the bf16 kernel, whose transposing V^T reads
  // want another).  A 16-byte LDS read serves lanes 0-7 with 16-23 (8-15
  // with 24-31, ...) in one 256-byte pass, an 8-byte one lanes 0-31, a
  // 16-byte write 8 lanes.  An operand read's pass takes chunk 4 kb + grp,
  // grp in {2i, 2i + 1}, of eight rows t: the rows start on the even slots
  // 2t (D = 128) or 10t (D = 64) mod 16, all distinct, and grp's low bit
  // fills the odd ones.  Chunk 4 kb + grp lies 64 kb bytes after chunk grp,
  // so a lane's reads take one address and immediate offsets.
  __device__ __forceinline__ static constexpr int kat(int t, int dc) { return t * kKRow + 16 * dc; }
  // the K chunk thread u converts: lanes 0-7 / 16-23 of each 32 take chunks
  // 0-7 / 8-15 of one row, lanes 8-15 / 24-31 those of the next (D = 128);
  // at D = 64 the four lane octets take chunks 0-7 of four rows.  Every
  // 16-byte write (8 lanes) then fills distinct slots of one row, and every
  // 8-byte read pass reads 256 contiguous bytes.
  __device__ __forceinline__ static int kconv_row(int u) {
    return D == 128 ? (u >> 5) * 2 + ((u >> 3) & 1)
                    : 4 * (u >> 5) + ((u >> 4) & 1) + 2 * ((u >> 3) & 1);
  }
  __device__ __forceinline__ static int kconv_chunk(int u) {
    return D == 128 ? (u & 7) | (((u >> 4) & 1) << 3) : u & 7;
  }
};

// N (4 or 2) 16-byte LDS reads at a + kOff + i kStride, waited for together
// (inline, for the reason given at read_vt_tr: a compiler-visible LDS read
// would first wait for the next tile's copies).
template <int N, int kOff, int kStride>
__device__ __forceinline__ void lds_read(uint32_t a, u32x4 (&r)[N]) {
  if constexpr (N == 4) {
    asm volatile(
        "ds_read_b128 %0, %4 offset:%5\n\t"
        "ds_read_b128 %1, %4 offset:%6\n\t"
        "ds_read_b128 %2, %4 offset:%7\n\t"
        "ds_read_b128 %3, %4 offset:%8\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
        : "v"(a), "i"(kOff), "i"(kOff + kStride), "i"(kOff + 2 * kStride),
          "i"(kOff + 3 * kStride));
  } else {
    static_assert(N == 2, "two or four operands");
    asm volatile(
        "ds_read_b128 %0, %2 offset:%3\n\t"
        "ds_read_b128 %1, %2 offset:%4\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1])
        : "v"(a), "i"(kOff), "i"(kOff + kStride));
  }
}

// Unit and dispatch order as in the bf16 prefill kernel (grid_order 0: unit
// x mod U; 1: unit x / nqt, a unit's tiles together; 2: the order of 1 cut
// into per-XCD contiguous runs).  Held to 168 registers: three workgroups
// per CU.
template <int D, bool PAGED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3)))
void prefill_i8_kernel(DecodeParams p) {
  using PG = I8PfGeo<D>;
  constexpr int KB = PG::KB, CB = PG::CB, NB = kCols / 16;
  __shared__ __align__(16) char smem[PG::kLds];

  const int R = p.R, T = p.T;
  const int64_t ncols = static_cast<int64_t>(T) * R;
  const int nqt = static_cast<int>((ncols + kRows - 1) / kRows);
  const int nsplit = p.n_splits;
  const int64_t units = static_cast<int64_t>(p.B) * p.G * nsplit;
  int64_t lin = blockIdx.x;
  if (p.grid_order == 2) {
    const int64_t nx = p.n_xcd, nwg = gridDim.x;
    const int64_t k = lin % nx, per = nwg / nx, rem = nwg % nx;
    lin = k * per + (k < rem ? k : rem) + lin / nx;
  }
  const int unit = static_cast<int>(p.grid_order == 0 ? lin % units : lin / nqt);
  const int qt = nqt - 1 - static_cast<int>(p.grid_order == 0 ? lin / units : lin % nqt);
  const int bg = unit / nsplit, split = unit - bg * nsplit;
  const int g = bg % p.G;
  const int b = p.grid_order == 2 && p.B <= 64 && p.B % p.n_xcd == 0 ? balanced_run_seq(p, bg / p.G)
                                                                      : bg / p.G;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, grp = lane >> 4;

  int L = scalar_load_i32(p.seq_lens + b);
  L = L < 0 ? 0 : (L > p.max_len_host ? p.max_len_host : L);
  const int win = L - T + 1;                      // query t sees the tokens j < win + t
  const int64_t c0 = static_cast<int64_t>(qt) * kRows;
  const int64_t c_last = (c0 + kRows < ncols ? c0 + kRows : ncols) - 1;
  int kmax = win + static_cast<int>(c_last / R);
  kmax = kmax < L ? kmax : L;
  const int64_t cw = c0 + wave * kCols;
  const int wbound = win + static_cast<int>((cw < ncols ? cw : c_last) / R);
  int k_lo = 0, k_hi = kmax;
  if (nsplit > 1) {
    if (split >= (L + p.chunk - 1) / p.chunk) return;
    k_lo = split * p.chunk;
    k_hi = k_lo + p.chunk < kmax ? k_lo + p.chunk : kmax;
  }

  int cbound[NB];
  int64_t qrow[NB];
  bool real[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int64_t c = cw + nb * 16 + n;
    real[nb] = c < ncols;
    const int t = static_cast<int>((real[nb] ? c : 0) / R);
    const int r = static_cast<int>((real[nb] ? c : 0) - static_cast<int64_t>(t) * R);
    cbound[nb] = real[nb] ? win + t : 0;
    qrow[nb] = (static_cast<int64_t>(b) * T + t) * p.H + g * R + r;
  }
  // q * scale * log2(e) * k_scale[g] rounded to fp16: lane (n, grp) of
  // block (nb, kb) holds dims kb*32 + grp*8 .. +7 of its row.  With the
  // K scale folded in, q . codes is the score itself.  An fp16 rounding
  // error is at most 2^-12 relative or 2^-25 absolute (below the normal
  // range), so the score is off by at most 2^-25 * 127 * D beyond the
  // relative part, whatever the scale.
  const float ksc = p.k_scale[g], vsc = p.v_scale[g];
  f16x8 qv[NB][KB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float* src = p.q_rot + qrow[nb] * D + grp * 8;
    const float qs = real[nb] ? p.qscale * ksc : 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const float4 x0 = *reinterpret_cast<const float4*>(src + kb * 32);
      const float4 x1 = *reinterpret_cast<const float4*>(src + kb * 32 + 4);
      const u32x4 h = {pack_f16(x0.x * qs, x0.y * qs), pack_f16(x0.z * qs, x0.w * qs),
                       pack_f16(x1.x * qs, x1.y * qs), pack_f16(x1.z * qs, x1.w * qs)};
      qv[nb][kb] = __builtin_bit_cast(f16x8, h);
    }
  }

  // The head's 16-token groups: group j16 of the sequence (contiguous: b's
  // row of S_max/16 groups; paged: the pool group the table gives, -1 when
  // its block id is outside the pool).
  const int64_t gstride = static_cast<int64_t>(p.G) * PG::kGroup;   // bytes per group
  // wave-uniform, so that the per-tile descriptor arithmetic stays scalar
  const char* kbase = reinterpret_cast<const char*>(uniform_u64(reinterpret_cast<uint64_t>(
      static_cast<const char*>(p.k) + static_cast<int64_t>(g) * PG::kGroup)));
  const char* vbase = reinterpret_cast<const char*>(uniform_u64(reinterpret_cast<uint64_t>(
      static_cast<const char*>(p.v) + static_cast<int64_t>(g) * PG::kGroup)));
  // One descriptor per half-tile group and operand: K spans the rows below
  // kmax (the others read as zeros), V^T the whole block of a valid group
  // (its tokens past kmax are masked, and codes are finite, so they add 0);
  // an invalid group reads as zeros without touching memory.
  struct TileSrc { rsrc_t k[2], v[2]; bool ok[2]; };
  auto tile_src = [&](int j0) {
    TileSrc ts;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int lo = j0 + 16 * h;
      int rows = __builtin_amdgcn_readfirstlane(kmax - lo);
      rows = rows < 0 ? 0 : (rows > 16 ? 16 : rows);
      int64_t grp16;
      ts.ok[h] = true;
      if (PAGED) {
        const int gi = rows > 0 ? paged_group(p, b, lo >> 4) : 0;
        if (gi < 0) { rows = 0; ts.ok[h] = false; }
        grp16 = gi < 0 ? 0 : gi;
      } else {
        grp16 = static_cast<int64_t>(b) * (p.max_seq_len >> 4) + (lo >> 4);
      }
      rows = __builtin_amdgcn_readfirstlane(rows);
      ts.k[h] = make_rsrc(kbase + grp16 * gstride, static_cast<uint32_t>(rows) * D);
      ts.v[h] = make_rsrc(vbase + grp16 * gstride, rows > 0 ? PG::kGroup : 0u);
    }
    return ts;
  };
  lds_char* const stage = (lds_char*)(smem);
  // this wave's copies: instructions wave + 4 i, each 1 KiB of one part
  // (K group 0, K group 1, V^T group 0, V^T group 1)
  auto issue = [&](const TileSrc& ts) {
#pragma unroll
    for (int i = 0; i < PG::NCI / kWaves; ++i) {
      const int jj = wave + kWaves * i;
      const int part = jj / (PG::kGroup / 1024);
      const uint32_t off = static_cast<uint32_t>((jj % (PG::kGroup / 1024)) * 1024 + lane * 16);
      const rsrc_t r = part == 0 ? ts.k[0] : part == 1 ? ts.k[1] : part == 2 ? ts.v[0] : ts.v[1];
      copy16_to_lds(r, stage + jj * 1024, off);
    }
  };
  // Convert the staged codes into the fp16 tile (all 256 threads).
  char* const kt16 = smem + PG::kStage;
  char* const vt16 = kt16 + PG::kKBytes;
  auto convert = [&]() {
    // K: chunk (t, dc) = 8 codes -> 16 bytes at kat(t, dc)
#pragma unroll
    for (int i = 0; i < kTT * PG::NDC / 256; ++i) {
      const int u = threadIdx.x + 256 * i;
      const int t = PG::kconv_row(u), dc = PG::kconv_chunk(u);
      const uint2 w = *reinterpret_cast<const uint2*>(smem + (t >> 4) * PG::kGroup +
                                                      (t & 15) * D + dc * 8);
      *reinterpret_cast<f16x8*>(kt16 + PG::kat(t, dc)) =
          codes_to_f16(w.x, w.y);
    }
    // V^T: dimension d of group h holds 16 codes, tokens 16 h + 0..15, as
    // four words of 4.  The fp16 row of d keeps them by class: class c (bytes
    // 16 c .. 16 c + 15) = word c of group 0, then word c of group 1, i.e.
    // tokens 4c .. 4c + 3 and 16 + 4c .. 16 + 4c + 3: the 8 tokens that lane
    // group c feeds to the P V matrix op, one 16-byte read.  codes_to_f16 of
    // (group 0 word c, group 1 word c) is class c as it stands.
    // Thread (wave wv, lane l) converts classes 2q, 2q + 1 of dimension d,
    // q = bit 2 of l, d = 32 wv + the other lane bits (l & 3, then bits 4, 3,
    // 5), and writes class 2q + q first.  16-byte writes are served 8 lanes
    // (128 bytes) at a time: lanes 0-7 hold dimensions 4 k .. 4 k + 3, whose
    // rows start 6 d mod 8 slots apart, each with q = 0 and 1, which write
    // slots of opposite parity.  The 16 lanes of a 16-byte read pass and the
    // 32 of an 8-byte one (the staged codes) also meet distinct banks.
    // Measured on a 32K prompt: no bank-conflict cycles (1.9e9 with the
    // dimensions in lane order).
    const int cl = threadIdx.x & 63, cw = threadIdx.x >> 6;
    const int d = 32 * cw + ((cl & 3) | (((cl >> 4) & 1) << 2) | (((cl >> 3) & 1) << 3) |
                             ((cl >> 5) << 4)),
              q = (cl >> 2) & 1;
    if (d < D) {
      lds_char* src = stage + 2 * PG::kGroup + d * 16 + 8 * q;   // group 0, words 2q, 2q + 1
      typedef const __attribute__((address_space(3))) uint64_t lds_u64;
      const uint64_t g0 = *reinterpret_cast<lds_u64*>(src);
      // opaque, so that the two reads are not fused into one two-address
      // read, which is served like a 16-byte read
      asm volatile("" : "+v"(src));
      const uint64_t g1 = *reinterpret_cast<lds_u64*>(src + PG::kGroup);   // group 1
      const uint32_t g0x = static_cast<uint32_t>(g0), g0y = static_cast<uint32_t>(g0 >> 32);
      const uint32_t g1x = static_cast<uint32_t>(g1), g1y = static_cast<uint32_t>(g1 >> 32);
      const uint32_t f0 = q ? g0y : g0x, f1 = q ? g1y : g1x;          // class 2q + q
      const uint32_t s0 = q ? g0x : g0y, s1 = q ? g1x : g1y;          // class 2q + 1 - q
      lds_char* const row = (lds_char*)(vt16) + d * PG::kVRow;
      *reinterpret_cast<__attribute__((address_space(3))) f16x8*>(row + 48 * q) =
          codes_to_f16(f0, f1);
      *reinterpret_cast<__attribute__((address_space(3))) f16x8*>(row + 16 + 16 * q) =
          codes_to_f16(s0, s1);
    }
  };

  // LDS read addresses, one per operand kind (the rest are immediate
  // offsets): K operand row 16 h2 + n, chunk kb*4 + grp at kaddr +
  // 16 h2 kKRow + 64 kb; V^T operand dimension 16 cb + n, tokens grp*8 .. +7
  // (class grp) at vaddr + 16 cb kVRow
  const uint32_t kaddr = lds_addr((lds_char*)(kt16)) + static_cast<uint32_t>(PG::kat(n, grp));
  const uint32_t vaddr = lds_addr((lds_char*)(vt16)) + static_cast<uint32_t>(n * PG::kVRow + grp * 16);
  static_assert(16 * PG::kKRow + 3 * 64 + 16 <= 65536 && (CB - 1) * 16 * PG::kVRow < 65536,
                "LDS read offsets fit the 16-bit offset field");

  f32x4 acc[NB][CB];
  float m[NB], lx[NB];
  // minus the reference the weights are taken against (the running max, 0
  // while there is none): the score MFMAs start from it and leave s - ref
  f32x4 nref[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    m[nb] = kNegInf; lx[nb] = 0.f;
    nref[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[nb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int nkt = k_hi > k_lo ? (k_hi + kTT - 1) / kTT : 0;
  const int kt_lo = k_lo / kTT;
  TileSrc cur;
  if (nkt > kt_lo) {
    cur = tile_src(kt_lo * kTT);
    issue(cur);
  }
  auto tile = [&](int kt, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int j0 = kt * kTT;
    vmem_wait<0>();                    // this wave's copies of tile kt have landed
    __syncthreads();                   // every wave's copies; the fp16 tile no longer read
    convert();
    __syncthreads();                   // the fp16 tile complete; the staged codes no longer read
    const TileSrc now = cur;
    if (kt + 1 < nkt) {
      cur = tile_src(j0 + kTT);
      issue(cur);
    }
    const bool masked = (MASK && j0 + kTT > wbound) || (PAGED && !(now.ok[0] && now.ok[1]));

    // S^T (raw, times k_scale below): token rows 16 h2 + 4 grp + j
    f32x4 s[NB][2];
    static_for<2>([&](auto h2c) {
      constexpr int h2 = decltype(h2c)::value;
      u32x4 kr[KB];
      lds_read<KB, 16 * h2 * PG::kKRow, 64>(kaddr, kr);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        f32x4 c = nref[nb];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          c = mfma_f16(__builtin_bit_cast(f16x8, kr[kb]), qv[nb][kb], c);
        s[nb][h2] = c;
      }
    });

    f16x8 pb[NB];
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
            const int t = j0 + 16 * h2 + 4 * grp + j;
            if (!(t < cbound[nb] && now.ok[h2])) sv[h2 * 4 + j] = kNegInf;
          }
      }
      // weights against the lazily kept running max (sv holds score - ref);
      // the tile's max only when a lane's sum passes 2^slack or the row has
      // no max yet (as in the bf16 prefill kernel)
      float e[8];
      float px = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        e[j] = __builtin_amdgcn_exp2f(sv[j]);
        px += e[j];
      }
      if (__builtin_expect(__any(!(px <= kRescaleBound) || m[nb] == kNegInf), 0)) {
        const float ref = -nref[nb][0];
        float mt = sv[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) mt = fmaxf(mt, sv[j]);
        mt = fmaxf(mt, __shfl_xor(mt, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float mn = fmaxf(m[nb], mt + ref);
        const float alpha = m[nb] == kNegInf ? 1.f : __builtin_amdgcn_exp2f(m[nb] - mn);
        lx[nb] *= alpha;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) acc[nb][cb] *= alpha;
        m[nb] = mn;
        const float ref2 = mn == kNegInf ? 0.f : mn;
        const float shift = ref - ref2;            // score - ref2 = sv + shift
        nref[nb] = f32x4{-ref2, -ref2, -ref2, -ref2};
        px = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          e[j] = __builtin_amdgcn_exp2f(sv[j] + shift);
          px += e[j];
        }
      }
      const u32x4 h = {pack_f16(e[0], e[1]), pack_f16(e[2], e[3]), pack_f16(e[4], e[5]),
                       pack_f16(e[6], e[7])};
      lx[nb] += px;
      pb[nb] = __builtin_bit_cast(f16x8, h);
    }

    // O^T[d][row] += V^T[d][t] P^T[t][row], four output blocks per read
    constexpr int NR = CB < 4 ? CB : 4;
    static_for<CB / NR>([&](auto c4c) {
      constexpr int c4 = NR * decltype(c4c)::value;
      u32x4 vr[NR];
      lds_read<NR, c4 * 16 * PG::kVRow, 16 * PG::kVRow>(vaddr, vr);
#pragma unroll
      for (int i = 0; i < NR; ++i)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[nb][c4 + i] = mfma_f16(__builtin_bit_cast(f16x8, vr[i]), pb[nb], acc[nb][c4 + i]);
    });
  };

  const int wg_bound = win + static_cast<int>(c0 / R);
  const int n_full = wg_bound >= kTT ? (wg_bound / kTT < nkt ? wg_bound / kTT : nkt) : 0;
  int kt = kt_lo;
  for (; kt < n_full; ++kt) tile(kt, std::false_type{});
  for (; kt < nkt; ++kt) tile(kt, std::true_type{});

#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    lx[nb] += __shfl_xor(lx[nb], 16);
    lx[nb] += __shfl_xor(lx[nb], 32);
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    if (!real[nb]) continue;
    const float inv = lx[nb] > 0.f ? vsc / lx[nb] : 0.f;
    const float lse2 = lx[nb] > 0.f ? m[nb] + log2f(lx[nb]) : kNegInf;
    float* dst;
    if (nsplit == 1) {
      dst = p.out + qrow[nb] * D + 4 * grp;
      if (grp == 0 && p.lse) p.lse[qrow[nb]] = lse2 * 0.69314718055994531f;
    } else {
      const int64_t slot = qrow[nb] * nsplit + split;
      dst = p.part_o + slot * D + 4 * grp;
      if (grp == 0) p.part_lse[slot] = lse2;
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
      *reinterpret_cast<f32x4*>(dst + 16 * cb) = acc[nb][cb] * inv;
  }
}

}  // namespace

hipError_t launch_prefill_i8(const DecodeParams& p_in, bool paged, const Launch& l) {
  DecodeParams p = p_in;
  if (p.T < 1 || p.R < 1 || (p.D != 64 && p.D != 128) || !p.k_scale || !p.v_scale)
    return hipErrorInvalidValue;
  if (!paged && p.max_seq_len % 16 != 0) return hipErrorInvalidValue;
  if (p.n_xcd < 1 || p.grid_order < -1 || p.grid_order > 2 || p.n_splits < 1)
    return hipErrorInvalidValue;
  if (p.n_splits > 1 && (p.chunk < kTT || p.chunk % kTT != 0 || !p.part_o || !p.part_lse))
    return hipErrorInvalidValue;
  const int64_t ncols = static_cast<int64_t>(p.T) * p.R;
  const int64_t nqt = (ncols + kRows - 1) / kRows;
  const int64_t units = static_cast<int64_t>(p.B) * p.G * p.n_splits;
  // grid_order -1 chooses: pairs fastest below n_xcd units; contiguous runs
  // per XCD when the runs are balanced by length (up to 64 sequences, a
  // multiple of n_xcd), or with key splits or more than 64 tiles per pair;
  // otherwise a pair's tiles together, round-robin over the XCDs, which
  // shares every pair's work evenly where unbalanced runs would not.  64
  // ragged sequences with 512-token chunks: 2.73 / 2.50 / 2.75 ms (orders
  // 0 / 1 / 2, runs not balanced), 2.54 (order 1) against 2.34 ms (balanced
  // runs); 2048-token chunks 9.13 against 8.09 ms.  A 32K prompt 58.8 / 63.8
  // / 58.8 ms.
  const bool balanced = p.B <= 64 && p.B % p.n_xcd == 0;
  if (p.grid_order < 0)
    p.grid_order = units < p.n_xcd ? 0 : (balanced || p.n_splits > 1 || nqt > 64 ? 2 : 1);
  const int64_t wgs = nqt * units;
  if (wgs <= 0 || wgs > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(wgs));
  void (*k)(DecodeParams) = p.D == 64 ? (paged ? prefill_i8_kernel<64, true> : prefill_i8_kernel<64, false>)
                                      : (paged ? prefill_i8_kernel<128, true> : prefill_i8_kernel<128, false>);
  return launch_kernel(k, grid, dim3(256), l, p);
}

}  // namespace kvd
