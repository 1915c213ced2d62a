// Causal prefill attention on the matrix cores: T new tokens per sequence (a
// prompt, or one chunk of it appended after a cached history), query t
// attending the tokens j < L_b - T + 1 + t.
//
// "Transformer推理核心：KV Cache、GQA与RoPE原理与工程实践" §4.2 describes the
// tiled attention that keeps score blocks on chip and carries an online
// softmax across key blocks; §5.1 b.v the causal mask.  Unlike the decode
// step, prefill is a dense contraction (every query row meets every key
// tile below its bound), so this kernel is organised for the MFMA pipe:
//
//  * a workgroup owns 128 query rows of one KV head -- the n_rep query heads
//    of 128 / n_rep consecutive new tokens -- and walks the key tiles below
//    their bounds, 32 tokens at a time;
//  * each key tile is copied HBM -> LDS once (every wave issues a quarter of
//    the copies, double-buffered, one barrier per tile) and read by all four
//    waves, each of which owns 32 of the rows: the GQA group shares every
//    tile, and no merge across waves is needed at the end;
//  * scores are computed transposed, S^T = K Q^T (v_mfma_f32_16x16x32_bf16,
//    A = K rows from LDS, B = the wave's q rows held in registers), so that
//    each query row's scores and accumulators live in one lane column and
//    the online softmax needs only two cross-lane shuffles;
//  * O^T = V^T P^T with V^T read from the staged tile (the decode kernel's
//    blocks, rows split in halves at D = 128) by the transposing LDS reads of
//    gfx950.
//
// Arithmetic: q (times scale * log2 e) and the probabilities enter the
// matrix cores rounded once to bf16, accumulation is fp32.  One running sum
// of the fp32 probabilities normalises the output and gives the
// log-sum-exp (the weights P V uses are those probabilities rounded to
// bf16, so the output is off by their rounding, 2^-9 relative at most).
// This is the precision of FlashAttention-2 in bf16; the decode kernels
// carry q and P as bf16 hi + lo pairs instead, at twice the matrix-core
// work, which the bandwidth-bound decode step does not notice but the
// compute-bound prefill would.
#include "mfma_tile.h"

namespace kvd {
namespace {

using namespace mt;

constexpr int kPfWaves = 4;
constexpr int kPfCols = 32;                      // query rows per wave (two column blocks)
constexpr int kPfRows = kPfWaves * kPfCols;      // query rows per workgroup
constexpr int kPfTT = 32;                        // key tokens per tile
constexpr float kRescaleBound = 256.f;           // 2^kRescaleSlack
static_assert(kRescaleSlack == 8.f, "kRescaleBound is 2^kRescaleSlack");
static_assert(kPfRows == kPrefillRows && kPfTT == kPrefillTile, "the host plans with these");

template <int D>
struct PfGeo {
  static constexpr int KB = D / 32;              // 32-dim blocks of the score contraction
  static constexpr int CB = D / 16;              // 16-dim blocks of the output
  static constexpr int NDC = D / 8;              // 16-byte chunks of a K row
  static constexpr int NKI = kPfTT * 2 * D / 1024;  // K copy instructions per tile
  // one K copy instruction's block (TPI rows), padded by 64 bytes at D = 128
  static constexpr bool kKPad = D == 128;
  static constexpr int kKBlock = kKPad ? 1024 + 64 : 1024;
  static constexpr int kKBytes = NKI * kKBlock;  // staged K tile
  static constexpr int TPI = 64 / NDC;           // K rows per copy instruction
  using VG = Geo<D>;                             // V copy blocks as in the decode kernel
  static constexpr int kVBytes = VG::kTileBytes;
  static constexpr int kBufBytes = kKBytes + kVBytes;
  static_assert(NKI % kPfWaves == 0 && VG::NVL % kPfWaves == 0, "copies split over the waves");
  // Chunk dc of K row t is stored at slot dc ^ swz(t) of the row, at byte
  // kat(t, dc).  A 16-byte LDS read serves lanes 0-7 together with lanes
  // 16-23 (8-15 with 24-31, and so on), 256 bytes per pass: a swizzle that
  // spread lanes 0-15 over the 64 banks left a 2-way conflict on every K
  // read (SQ_LDS_BANK_CONFLICT).  Such a pass reads chunks 4 kb + grp, grp in
  // {2i, 2i + 1}, of the eight rows tile_row(n), n < 8 (or n >= 8).  At
  // D = 128 those rows are 4 m + r, m = 0..3, r in {0, 1} (or {2, 3}): the
  // 64-byte block padding puts the four m on four different 64-byte quarters
  // of the banks, and swz = 2 (t & 1) with grp's low bit gives the four
  // slots of a quarter.  swz leaves bits 2-3 of the chunk alone, so chunk
  // 4 kb + grp of a row lies 64 kb bytes after chunk grp: one address and
  // immediate offsets serve a lane's reads.  At D = 64 (128-byte rows, no
  // padding) swz sends the rows to four slots per 128-byte half.
  __device__ __forceinline__ static int swz(int t) {
    return D == 128 ? (t & 1) << 1 : ((t >> 1) & 6);
  }
  __device__ __forceinline__ static int kat(int t, int dc) {
    return (t / TPI) * kKBlock + (t % TPI) * (2 * D) + 16 * (dc ^ swz(t));
  }
  // Staged V: blocks of one copy instruction each (RPI rows, 32 bytes of
  // padding after every block, so blocks start 8 banks apart).  At D = 128 a
  // block holds the first 128 bytes of its four rows, then their second 128
  // bytes.  The transposing reads of lanes 0-31 (lane groups 0 and 1) go out
  // together and address rows 4 m + grp of four blocks: with whole 256-byte
  // rows, group 1's rows sat on the same 32 banks as group 0's (a 2-way
  // conflict on every V^T read); with split rows they are 128 bytes apart and
  // the eight rows cover all 64 banks.
  static constexpr bool kVSplit = D == 128;
  __device__ __forceinline__ static constexpr int vat(int r, int c) {
    return kVSplit ? (r / VG::RPI) * VG::BLOCK + (c >> 7) * 512 + (r % VG::RPI) * 128 + (c & 127)
                   : VG::at(r, c);
  }
  // row (within its block) and byte (within its row) copied by lane l of a
  // V copy instruction, which lands 16 bytes at block + 16 l
  __device__ __forceinline__ static int vrow_of(int l) { return kVSplit ? (l >> 3) & 3 : l / VG::LPR; }
  __device__ __forceinline__ static int vbyte_of(int l) {
    return kVSplit ? (l >> 5) * 128 + (l & 7) * 16 : (l % VG::LPR) * 16;
  }
};

// Four (D = 128) or two (D = 64) 16-byte K operands from LDS, waiting for
// their own reads.  Inline assembly for the reason given at read_vt_tr: a
// compiler-visible LDS read would first wait for the next tile's copies.
template <int kOff>
__device__ __forceinline__ void read_k(const uint32_t (&a)[4], bf16x8 (&k)[4]) {
  u32x4 r0, r1, r2, r3;
  asm volatile(
      "ds_read_b128 %0, %4 offset:%8\n\t"
      "ds_read_b128 %1, %5 offset:%8\n\t"
      "ds_read_b128 %2, %6 offset:%8\n\t"
      "ds_read_b128 %3, %7 offset:%8\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "i"(kOff));
  k[0] = __builtin_bit_cast(bf16x8, r0);
  k[1] = __builtin_bit_cast(bf16x8, r1);
  k[2] = __builtin_bit_cast(bf16x8, r2);
  k[3] = __builtin_bit_cast(bf16x8, r3);
}
// The same four reads from one address, 64 bytes apart (D = 128).
template <int kOff>
__device__ __forceinline__ void read_k(uint32_t a, bf16x8 (&k)[4]) {
  u32x4 r0, r1, r2, r3;
  asm volatile(
      "ds_read_b128 %0, %4 offset:%5\n\t"
      "ds_read_b128 %1, %4 offset:%6\n\t"
      "ds_read_b128 %2, %4 offset:%7\n\t"
      "ds_read_b128 %3, %4 offset:%8\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
      : "v"(a), "i"(kOff), "i"(kOff + 64), "i"(kOff + 128), "i"(kOff + 192));
  k[0] = __builtin_bit_cast(bf16x8, r0);
  k[1] = __builtin_bit_cast(bf16x8, r1);
  k[2] = __builtin_bit_cast(bf16x8, r2);
  k[3] = __builtin_bit_cast(bf16x8, r3);
}
template <int kOff>
__device__ __forceinline__ void read_k(const uint32_t (&a)[2], bf16x8 (&k)[2]) {
  u32x4 r0, r1;
  asm volatile(
      "ds_read_b128 %0, %2 offset:%4\n\t"
      "ds_read_b128 %1, %3 offset:%4\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1)
      : "v"(a[0]), "v"(a[1]), "i"(kOff));
  k[0] = __builtin_bit_cast(bf16x8, r0);
  k[1] = __builtin_bit_cast(bf16x8, r1);
}

// Workgroup x owns one query-row tile of one unit -- a (sequence, KV head)
// pair, or with key splits a (pair, split) -- whose tiles go most keys
// first.  U units in all.  grid_order 0: unit x mod U, tile nqt - 1 - x / U.
// 1: unit x / nqt, tile nqt - 1 - x mod nqt (a unit's tiles together).
// 2: the order of 1 cut into n_xcd contiguous runs, run k taken by the
// workgroups x = k mod n_xcd, which the device sends to one XCD, so that a
// unit's tiles, which all read its keys, share one L2; with up to 64
// sequences, a multiple of n_xcd, the list's sequences are ordered so that
// the runs hold equal shares of the work (balanced_run_seq).  Held to 168
// registers, three workgroups share a CU (measured 18% faster than two).
template <int D, bool PAGED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3)))
void prefill_kernel(DecodeParams p) {
  using PG = PfGeo<D>;
  using VG = Geo<D>;
  constexpr int KB = PG::KB, CB = PG::CB, NB = kPfCols / 16;
  __shared__ __align__(16) char smem[2 * PG::kBufBytes];

  const int R = p.R, T = p.T;
  const int64_t ncols = static_cast<int64_t>(T) * R;
  const int nqt = static_cast<int>((ncols + kPfRows - 1) / kPfRows);
  const int nsplit = p.n_splits;                   // 1: no key split
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
  const int64_t c0 = static_cast<int64_t>(qt) * kPfRows;
  const int64_t c_last = (c0 + kPfRows < ncols ? c0 + kPfRows : ncols) - 1;
  // keys any row of the workgroup sees; the smallest bound of this wave's rows
  int kmax = win + static_cast<int>(c_last / R);
  kmax = kmax < L ? kmax : L;
  const int64_t cw = c0 + wave * kPfCols;
  const int wbound = win + static_cast<int>((cw < ncols ? cw : c_last) / R);
  // this workgroup's keys [k_lo, k_hi): a split's whole tiles.  A split at
  // or past the sequence's end writes nothing (the merge reads only the
  // splits that hold its tokens); one below it writes every row, empty
  // ones as (0, -inf).
  int k_lo = 0, k_hi = kmax;
  if (nsplit > 1) {
    if (split >= (L + p.chunk - 1) / p.chunk) return;
    k_lo = split * p.chunk;
    k_hi = k_lo + p.chunk < kmax ? k_lo + p.chunk : kmax;
  }

  // the lane's query rows: column nb*16 + n of the wave
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
  // q * scale * log2(e) rounded to bf16: lane (n, grp) of block (nb, kb)
  // holds dims kb*32 + grp*8 .. +7 of its row
  bf16x8 qv[NB][KB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float* src = p.q_rot + qrow[nb] * D + grp * 8;
    const float qs = real[nb] ? p.qscale : 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const float4 x0 = *reinterpret_cast<const float4*>(src + kb * 32);
      const float4 x1 = *reinterpret_cast<const float4*>(src + kb * 32 + 4);
      const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      const u32x4 h = {pack_bf16(xv[0] * qs, xv[1] * qs), pack_bf16(xv[2] * qs, xv[3] * qs),
                       pack_bf16(xv[4] * qs, xv[5] * qs), pack_bf16(xv[6] * qs, xv[7] * qs)};
      qv[nb][kb] = __builtin_bit_cast(bf16x8, h);
    }
  }

  // bytes between consecutive tokens of one KV head, and the start of this
  // (sequence, KV head) -- of KV head g of the pool when paged
  const int64_t rs = static_cast<int64_t>(p.G) * (2 * D);
  const int64_t head0 = (PAGED ? 0 : static_cast<int64_t>(b) * p.max_seq_len * rs) +
                        static_cast<int64_t>(g) * (2 * D);
  // wave-uniform, so that the per-tile descriptor arithmetic stays scalar
  const char* kbase = reinterpret_cast<const char*>(
      uniform_u64(reinterpret_cast<uint64_t>(static_cast<const char*>(p.k) + head0)));
  const char* vbase = reinterpret_cast<const char*>(
      uniform_u64(reinterpret_cast<uint64_t>(static_cast<const char*>(p.v) + head0)));

  // One descriptor per 16-token half of a tile and operand, spanning the
  // valid rows (below kmax, in a valid block): other rows read as zeros
  // without touching memory.
  struct TileSrc { rsrc_t k[2], v[2]; bool ok[2]; };
  auto tile_src = [&](int j0) {
    TileSrc ts;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int lo = j0 + 16 * h;
      int rows = __builtin_amdgcn_readfirstlane(kmax - lo);
      rows = rows < 0 ? 0 : (rows > 16 ? 16 : rows);
      int64_t off;
      ts.ok[h] = true;
      if (PAGED) {
        const int blk = rows > 0 ? paged_group(p, b, lo >> 4) : 0;
        if (blk < 0) { rows = 0; ts.ok[h] = false; }
        off = static_cast<int64_t>(blk < 0 ? 0 : blk) * 16 * rs;
      } else {
        off = static_cast<int64_t>(lo) * rs;
      }
      rows = __builtin_amdgcn_readfirstlane(rows);
      const uint32_t bytes = static_cast<uint32_t>(rows) * static_cast<uint32_t>(rs);
      ts.k[h] = make_rsrc(kbase + off, bytes);
      ts.v[h] = make_rsrc(vbase + off, bytes);
    }
    return ts;
  };
  // this wave's quarter of a tile's copies: K instructions wave + 4 i (each
  // 64 16-byte chunks, rows jj * TPI ..), V instructions likewise (rows
  // jj * RPI .., placed by vrow_of / vbyte_of)
  uint32_t koffc[PG::NKI / kPfWaves];
#pragma unroll
  for (int i = 0; i < PG::NKI / kPfWaves; ++i) {
    const int jj = wave + kPfWaves * i;
    const int u = jj * 64 + lane;
    const int t = u / PG::NDC, slot = u % PG::NDC;
    const int dc = slot ^ PG::swz(t);
    koffc[i] = static_cast<uint32_t>((t & 15) * rs + dc * 16);
  }
  const uint32_t vlane = static_cast<uint32_t>(PG::vrow_of(lane) * rs + PG::vbyte_of(lane));
  lds_char* const buf0 = (lds_char*)(smem);
  auto issue = [&](const TileSrc& ts, int sel) {
    lds_char* kb_ = buf0 + sel * PG::kBufBytes;
#pragma unroll
    for (int i = 0; i < PG::NKI / kPfWaves; ++i) {
      const int jj = wave + kPfWaves * i;
      const int h = (jj * PG::TPI) >> 4;
      copy16_to_lds(h == 0 ? ts.k[0] : ts.k[1], kb_ + jj * PG::kKBlock, koffc[i]);
    }
#pragma unroll
    for (int i = 0; i < VG::NVL / kPfWaves; ++i) {
      const int jj = wave + kPfWaves * i;
      const int h = (jj * VG::RPI) >> 4;
      const uint32_t off = vlane + static_cast<uint32_t>(((jj * VG::RPI) & 15) * rs);
      copy16_to_lds(h == 0 ? ts.v[0] : ts.v[1], kb_ + PG::kKBytes + jj * VG::BLOCK, off);
    }
  };
  // V rows this wave copied that hold no valid token become zeros (an
  // out-of-range copy leaves LDS as it was, and 0 * stale must stay 0)
  auto zero_invalid_v = [&](const TileSrc& ts, int j0, int sel) {
    const uint32_t vb = lds_addr(buf0 + sel * PG::kBufBytes + PG::kKBytes);
#pragma unroll
    for (int i = 0; i < VG::NVL / kPfWaves; ++i) {
      const int jj = wave + kPfWaves * i;
      const int r = jj * VG::RPI + PG::vrow_of(lane);
      const bool ok = (jj * VG::RPI) >> 4 == 0 ? ts.ok[0] : ts.ok[1];
      if (!(j0 + r < kmax && ok)) lds_zero16(vb + jj * VG::BLOCK + lane * 16);
    }
  };

  // LDS read offsets of the lane's K operands: row 16 h2 + tile_row(n), chunk
  // kb*4 + grp; at D = 128 one offset, the rest 4 kKBlock h2 + 64 kb further
  constexpr int NKO = PG::kKPad ? 1 : 2 * KB;
  uint32_t koff[NKO];
#pragma unroll
  for (int i = 0; i < NKO; ++i) {
    const int h2 = i / KB, kb = i % KB;
    koff[i] = lds_addr(buf0) + static_cast<uint32_t>(PG::kat(16 * h2 + tile_row(n), kb * 4 + grp));
  }
  // the lane's address for read_vt_tr: row tile_row(4 grp + n / 4), dims 4 (n % 4) ..
  const uint32_t vrd = static_cast<uint32_t>(PG::vat(tile_row(4 * grp + n / 4), 8 * (n % 4)));
  constexpr int kVHalf = (16 / VG::RPI) * VG::BLOCK;     // rows r -> r + 16

  f32x4 acc[NB][CB];
  float m[NB], lx[NB];
  // minus the reference the weights are taken against (the running max, 0
  // while there is none), in all four lanes of a score accumulator: the
  // score MFMAs start from it and leave s - ref
  f32x4 nref[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    m[nb] = kNegInf; lx[nb] = 0.f;
    nref[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[nb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // key tiles [kt_lo, nkt)
  const int nkt = k_hi > k_lo ? (k_hi + kPfTT - 1) / kPfTT : 0;
  const int kt_lo = k_lo / kPfTT;
  TileSrc cur;
  if (nkt > kt_lo) {
    cur = tile_src(kt_lo * kPfTT);
    issue(cur, kt_lo & 1);
  }
  // One key tile: wait for its copies, request the next tile's, then scores,
  // online softmax and P V.  MASK (a constant at each call) says whether the
  // tile may reach past a row's bound or hold an invalid block.
  auto tile = [&](int kt, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int j0 = kt * kPfTT;
    const int sel = kt & 1;
    vmem_wait<0>();                    // this wave's copies of tile kt have landed
    if (j0 + kPfTT > kmax || !cur.ok[0] || !cur.ok[1]) zero_invalid_v(cur, j0, sel);
    __syncthreads();                   // every wave's copies of tile kt; tile kt - 1 no longer read
    const TileSrc now = cur;
    if (kt + 1 < nkt) {
      cur = tile_src(j0 + kPfTT);
      issue(cur, sel ^ 1);
    }
    const uint32_t kaddr = static_cast<uint32_t>(sel * PG::kBufBytes);
    const uint32_t vaddr = lds_addr(buf0) + kaddr + PG::kKBytes + vrd;
    // wave-uniform; an invalid block (paged) masks its tokens on either path
    const bool masked = (MASK && j0 + kPfTT > wbound) || (PAGED && !(now.ok[0] && now.ok[1]));

    // S^T - ref: token rows 16 h2 + 4 grp + j, lane column n of block nb
    f32x4 s[NB][2];
    static_for<2>([&](auto h2c) {
      constexpr int h2 = decltype(h2c)::value;
      bf16x8 ka[KB];
      if constexpr (PG::kKPad) {
        read_k<h2 * 4 * PG::kKBlock>(kaddr + koff[0], ka);
      } else {
        uint32_t a[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) a[kb] = kaddr + koff[h2 * KB + kb];
        read_k<0>(a, ka);
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        f32x4 c = nref[nb];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) c = mfma(ka[kb], qv[nb][kb], c);
        s[nb][h2] = c;
      }
    });

    bf16x8 pb[NB];
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
            const int t = j0 + 16 * h2 + tile_row(4 * grp + j);
            if (!(t < cbound[nb] && now.ok[h2])) sv[h2 * 4 + j] = kNegInf;
          }
      }
      // Probabilities against the running max (lazily kept: it moves only
      // when a score passes it by more than kRescaleSlack); sv already holds
      // score - ref.  A lane's sum of its 8 weights bounds each of them, so
      // the tile's max is needed only when that sum passes 2^slack (or is not
      // finite), or while the row has no max yet: then the max moves to the
      // tile's, the state is rescaled and the weights are taken again.
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
      u32x4 h;
#pragma unroll
      for (int j = 0; j < 4; ++j) h[j] = pack_bf16(e[2 * j], e[2 * j + 1]);
      lx[nb] += px;
      pb[nb] = __builtin_bit_cast(bf16x8, h);
    }

    // O^T[d][row] += V^T[d][t] P^T[t][row]
    static_for<CB>([&](auto cbc) {
      constexpr int cb = decltype(cbc)::value;
      const bf16x8 av = read_vt_tr<PG::vat(0, 32 * cb), kVHalf>(vaddr);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[nb][cb] = mfma(av, pb[nb], acc[nb][cb]);
    });
  };

  // Tiles below the workgroup's smallest bound need no causal mask; the
  // rest, at most two per wave, take the masked body.
  const int wg_bound = win + static_cast<int>(c0 / R);
  const int n_full = wg_bound >= kPfTT ? (wg_bound / kPfTT < nkt ? wg_bound / kPfTT : nkt) : 0;
  int kt = kt_lo;
  for (; kt < n_full; ++kt) tile(kt, std::false_type{});
  for (; kt < nkt; ++kt) tile(kt, std::true_type{});

  // the four lane groups of a column hold partial sums under one max
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    lx[nb] += __shfl_xor(lx[nb], 16);
    lx[nb] += __shfl_xor(lx[nb], 32);
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    if (!real[nb]) continue;
    const float inv = lx[nb] > 0.f ? 1.f / lx[nb] : 0.f;
    const float lse2 = lx[nb] > 0.f ? m[nb] + log2f(lx[nb]) : kNegInf;
    if (nsplit == 1) {
      float* dst = p.out + qrow[nb] * D + 4 * grp;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
        *reinterpret_cast<f32x4*>(dst + 16 * cb) = acc[nb][cb] * inv;
      if (grp == 0 && p.lse) p.lse[qrow[nb]] = lse2 * 0.69314718055994531f;
    } else {
      // the split's partial: normalised output and log2-sum-exp
      const int64_t slot = qrow[nb] * nsplit + split;
      float* dst = p.part_o + slot * D + 4 * grp;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
        *reinterpret_cast<f32x4*>(dst + 16 * cb) = acc[nb][cb] * inv;
      if (grp == 0) p.part_lse[slot] = lse2;
    }
  }
}

}  // namespace

// grid_order -1 chooses.  Fewer (sequence, KV head) pairs than XCDs: pairs
// fastest, which deals every pair's tiles over the XCDs.  Otherwise a pair's
// query tiles go together in contiguous runs per XCD, so that a pair's keys
// are fetched into one L2 instead of eight.  Measured on 64 ragged sequences
// with 8 KV heads (orders 0 / 1 / 2, runs in batch order): 512-token chunks
// 3.63 / 2.87 / 2.37 ms, 2048-token chunks 12.2 / 8.79 / 8.57 ms, 8192-token
// chunks 54.0 / 40.2 / 34.3 ms; a 32K prompt with 32 KV heads 63.3 / 68.9 /
// 59.5 ms.  Runs in batch order left one XCD a fifth more work than the
// mean on that batch; balanced by length (balanced_run_seq) the 512-token
// chunks take 2.08 ms (order 1: 2.88), the 2048-token chunks 7.35 ms.
hipError_t launch_prefill_mfma(const DecodeParams& p_in, bool paged, const Launch& l) {
  DecodeParams p = p_in;
  if (p.T < 1 || p.R < 1 || (p.D != 64 && p.D != 128)) return hipErrorInvalidValue;
  if (p.n_xcd < 1 || p.grid_order < -1 || p.grid_order > 2 || p.n_splits < 1) return hipErrorInvalidValue;
  if (p.n_splits > 1 && (p.chunk < kPfTT || p.chunk % kPfTT != 0 || !p.part_o || !p.part_lse))
    return hipErrorInvalidValue;
  const int64_t ncols = static_cast<int64_t>(p.T) * p.R;
  const int64_t nqt = (ncols + kPfRows - 1) / kPfRows;
  const int64_t units = static_cast<int64_t>(p.B) * p.G * p.n_splits;
  // with key splits the units hold equal key counts: runs per XCD
  if (p.grid_order < 0)
    p.grid_order = units < p.n_xcd ? 0 : 2;
  const int64_t wgs = nqt * units;
  if (wgs <= 0 || wgs > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(wgs));
  void (*k)(DecodeParams) = p.D == 64 ? (paged ? prefill_kernel<64, true> : prefill_kernel<64, false>)
                                      : (paged ? prefill_kernel<128, true> : prefill_kernel<128, false>);
  return launch_kernel(k, grid, dim3(256), l, p);
}

}  // namespace kvd
