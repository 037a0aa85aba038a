// Dense contractions of the DoRA hot path on gfx950.
//
// bf16 operands run on the CDNA4 matrix cores (v_mfma_f32_32x32x16_bf16,
// float32 accumulation); float32 layers use v_mfma_f32_32x32x2_f32 tiles.  One kernel
// template covers every contraction of the path:
//   C[m, n] = alpha * sum over segments s, k < K_s of opA_s(m, k) * opB_s(n, k)
// where each operand is either K-contiguous or M/N-contiguous in memory, and
// up to three K segments are concatenated (e.g. [x | xs] . [W0 | B]^T).
//
// Tiling.  A workgroup owns a BM x BN output tile and walks K in 64-deep
// steps through two LDS stages.  LDS rows are 64 bf16 = 128 B, split in eight
// 16-byte chunks whose order is XOR-swizzled by the row index
// ((row & 7) ^ ((row >> 3) & 7)) so that the eight (and sixteen) rows a
// 16-byte-per-lane read or write touches land in distinct bank groups.
// Both operand layouts go global -> LDS directly (buffer_load ... lds).
// K-contiguous operands keep their rows and are read with ds_read_b128;
// M/N-contiguous operands keep their k-major layout (chunks swizzled by the
// k-row instead) and are read with the transposing ds_read_b64_tr_b16, which
// yields the same MFMA fragments.  (Tiles narrower than 128 rows transpose
// M/N-contiguous operands in registers instead.)  Each wave computes a
// (BM/WM) x (BN/WN) sub-tile of 32x32 MFMA blocks.  The MFMA runs as
// D = opB-tile x opA-tile^T so that every lane ends up holding four
// consecutive output columns.
//
// Instruction budget.  With eight waves per CU every scalar or vector
// instruction of the K loop competes with the MFMA issue, so the loop holds
// little else: buffer descriptors and per-lane offsets are set once per K
// segment, the K position travels in the scalar offset of each load, only a
// segment's last partial step checks K per lane, and fragment reads are
// per-lane bases plus immediate offsets (the stage loop is unrolled by two).
//
// Workgroups are dispatched round-robin over the 8 XCDs; the tile index is
// remapped so that consecutive tiles (which share operand panels) run on
// one XCD and share its L2, and tiles are walked in groups of tile-rows sized
// so that each XCD holds a compact block (tile_coords).
#include <algorithm>

#include "kernels.h"
#include "common.h"

namespace dora {
namespace {

constexpr int kBK = 64;           // K depth of one LDS stage (bf16)
constexpr int kRowBytes = kBK * 2;

struct KArgs {
  int M, N;
  int nseg;
  const uint16_t* a[3];
  const uint16_t* b[3];
  int64_t lda[3], ldb[3];
  int K[3];
  int kt_end[3];         // cumulative number of K tiles after each segment
  int kt_total;          // kt_end[nseg - 1], kept apart so no array is indexed at run time
  int kt_per_split;
  int tiles_m, tiles_n;
  void* c;
  int64_t ldc;
  int64_t split_stride;
  float alpha;
  const void* mag;
  const float* norm;
  const void* add;
  int64_t ld_add;
  float* rowsq;          // kEpiNorm: [nsplit][M] sums of squares of opA over segment 0
  float* rowdot;         // kEpiNorm: [nsplit][tiles_n][M] row dots of alpha*C with `add`
  float* norm_out;       // kEpiNorm: row norms written by the last workgroup of each tile row
  uint32_t* done;        // kEpiNorm: [tiles_m] arrival counters, zero at launch
  int nsplit;            // K splits (the bf16 kernels' grid is tiles x nsplit, 1-D)
};

__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 7); }

// ---- buffer resources ---------------------------------------------------------
// Operands are read through raw buffer resources rebased at the current tile,
// so out-of-range rows (and K tails, sent to kOob) come back as zeros from the
// hardware range check instead of through branches.
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr uint32_t kOob = 0x80000000u;   // offset beyond every record: the load returns 0
constexpr int kRsrcWord3 = 0x00020000;   // raw (untyped) buffer, gfx9-family data format

// `base` and `bytes` must be wave-uniform: they are read from the first lane so
// that the descriptor always lives in scalar registers (a descriptor the
// compiler believes divergent would be wrapped in a per-lane loop).
__device__ __forceinline__ Rsrc make_rsrc(const void* base, int64_t bytes) {
  const int64_t b = bytes < 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : bytes);
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const int nb = __builtin_amdgcn_readfirstlane((int)b);
  void* ub = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, nb, kRsrcWord3);
}
__device__ __forceinline__ u32x4 bload16(Rsrc r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// ---- operand copiers ---------------------------------------------------------
// Both keep their descriptor and per-lane offsets for a whole K segment; a
// 64-deep step only supplies the scalar offset of its K position.

// K-contiguous operand, R rows x 64 k per stage, copied straight into LDS with
// buffer_load ... lds: one wave instruction fills 8 rows x 128 B, lane l takes
// row l/8 and physical chunk l%8, i.e. logical chunk (l%8) ^ swz(row).  Every
// instruction has its own per-lane offset (its row and chunk), set once per
// segment, and a step only supplies the K position as the scalar offset.  The
// hardware range check covers the per-lane offset only (the scalar offset is
// added after it), so rows past the operand, beyond the descriptor's records,
// read as zeros, and the K position (< ld) keeps a valid row inside its row.
template <int R, int NW>
struct CopyKC {
  static constexpr int kInstr = R / 8 / NW;   // 16-byte copies per lane and stage
  static_assert(R % (8 * NW) == 0, "rows must split evenly over the waves");
  // Per-lane offsets reach (R - 1) * ld * 2 + 112; the planner keeps R * ld * 2
  // below 2^31 (always true for R <= 256, since every stride is below 2^22).
  static_assert(R <= 384, "tile rows");
  Rsrc rs;                 // tile base at k = 0, records = valid rows * ld * 2
  uint32_t off[kInstr];    // row * ld * 2 + chunk * 16
  __device__ __forceinline__ static int row_of(int i, int wave, int lane) {
    return (wave + i * NW) * 8 + (lane >> 3);
  }
  __device__ __forceinline__ void prepare(const uint16_t* p, int64_t ld, int row0, int nrows, int,
                                          int wave, int lane, int) {
    int64_t rows = nrows - row0;
    if (rows > R) rows = R;
    rs = make_rsrc(p + (int64_t)row0 * ld, rows * ld * 2);
#pragma unroll
    for (int i = 0; i < kInstr; ++i) {
      const int row = row_of(i, wave, lane);
      const int kc = (lane & 7) ^ swz(row);
      off[i] = (uint32_t)row * (uint32_t)(ld * 2) + (uint32_t)kc * 16u;
    }
  }
  // Step kt (relative to the segment) into the stage tile.  On a partial step
  // the chunks at or beyond K read as zeros: kOob plus the scalar offset stays
  // below 2^32 and beyond every record count.
  template <bool TAIL>
  __device__ __forceinline__ void issue(uint8_t* lds_tile, int kt, int K, int wave, int lane,
                                        int) {
    const int kbytes = kt * kRowBytes;
#pragma unroll
    for (int i = 0; i < kInstr; ++i) {
      uint32_t o = off[i];
      if (TAIL) {
        const int row = row_of(i, wave, lane);
        const int kc = (lane & 7) ^ swz(row);
        if (kt * kBK + kc * 8 >= K) o = kOob;
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(lds_tile + (wave + i * NW) * 8 * kRowBytes),
          16, (int)o, kbytes, 0, 0);
    }
  }
  __device__ __forceinline__ void commit(uint8_t*, int) {}
};

// M/N-contiguous operand: element (row, k) at p[k*ld + row].  Copied as blocks
// of 4 consecutive k x 8 consecutive rows (four 16-byte loads), transposed in
// registers into eight 8-byte row pieces.  Columns past the operand carry kOob
// from the start; rows k past K are masked on a segment's last step only.
template <int R, int NT>
struct CopyMC {
  static constexpr int kRowChunks = R / 8;
  static constexpr int kBlocks = kRowChunks * (kBK / 4);
  static constexpr int kPer = (kBlocks + NT - 1) / NT;
  static_assert(kRowChunks % 8 == 0, "block order assumes a multiple of 64 rows");
  // Block b -> (k-quad kq, row-chunk rc): eight consecutive blocks take eight
  // consecutive row chunks and the next eight the other half of the same
  // 16-byte k chunk, so sixteen lanes' 8-byte LDS writes fill sixteen distinct
  // bank slots, while each eight lanes still read 128 contiguous bytes.
  __device__ __forceinline__ static void block_of(int b, int& kq, int& rc) {
    const int lo = b & 7, kh = (b >> 3) & 1, rest = b >> 4;
    constexpr int kHi = kRowChunks / 8;
    rc = (rest % kHi) * 8 + lo;
    kq = (rest / kHi) * 2 + kh;
  }
  Rsrc rs;
  const uint16_t* base;    // column row0, k = kbase
  int64_t ld;
  int kt_base;             // step the descriptor starts at
  int kt_span;             // steps one descriptor covers with a 31-bit scalar offset
  uint32_t off[kPer];      // kq*4 * ld * 2 + rc * 16, or kOob; k row j adds j * ld * 2
  u32x4 v[kPer][4];
  __device__ __forceinline__ void prepare(const uint16_t* p, int64_t ldv, int row0, int nrows,
                                          int K, int, int, int tid) {
    base = p + row0;
    ld = ldv;
    kt_base = 0;
    kt_span = (int)((int64_t)0x40000000 / (ldv * 2 * kBK));   // >= 2: ld < 2^22
    rs = make_rsrc(base, (int64_t)K * ldv * 2);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int b = tid + i * NT;
      int kq, rc;
      block_of(b, kq, rc);
      const bool ok = (kBlocks % NT == 0 || b < kBlocks) && row0 + rc * 8 < nrows;
      off[i] = ok ? (uint32_t)(kq * 4) * (uint32_t)(ldv * 2) + (uint32_t)rc * 16u : kOob;
    }
  }
  template <bool TAIL>
  __device__ __forceinline__ void issue(uint8_t*, int kt, int K, int, int, int tid) {
    if (kt - kt_base >= kt_span) {   // keep the scalar offset below 2^30
      kt_base = kt;
      rs = make_rsrc(base + (int64_t)kt * kBK * ld, (int64_t)(K - kt * kBK) * ld * 2);
    }
    const int ld2 = (int)(ld * 2);
    const int soff = (kt - kt_base) * kBK * ld2;   // < 2^30; plus 3 * ld2 < 2^31
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      int kq = 0, rc = 0;
      if (TAIL) block_of(tid + i * NT, kq, rc);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t o = off[i];
        if (TAIL && kt * kBK + kq * 4 + j >= K) o = kOob;
        v[i][j] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)o, soff + j * ld2, 0));
      }
    }
  }
  __device__ __forceinline__ void commit(uint8_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int b = tid + i * NT;
      if (kBlocks % NT != 0 && b >= kBlocks) continue;
      int kq, rc;
      block_of(b, kq, rc);
      const int chunk = kq >> 1, half = kq & 1;
#pragma unroll
      for (int mm = 0; mm < 8; ++mm) {
        const int d = mm >> 1;
        const uint32_t a0 = v[i][0][d], a1 = v[i][1][d], a2 = v[i][2][d], a3 = v[i][3][d];
        // bf16 element mm&1 of each of the four k rows, paired by byte permutes
        const uint32_t sel = (mm & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t lo = __builtin_amdgcn_perm(a1, a0, sel);
        const uint32_t hi = __builtin_amdgcn_perm(a3, a2, sel);
        const int row = rc * 8 + mm;
        *reinterpret_cast<u32x2*>(lds + row * kRowBytes + ((chunk ^ swz(row)) << 4) + half * 8) =
            u32x2{lo, hi};
      }
    }
  }
};

// M/N-contiguous operand copied straight into LDS (buffer_load ... lds) in
// its own k-major layout: a stage is 64 k-rows of R elements (2R bytes), the
// 16-byte chunks of k-row k XOR-swizzled by 4*(k % 4).  The stage's chunks are
// numbered row by row, c = k-row * kLPR + chunk, and sit at byte 16 c of the
// stage, so one wave instruction fills the 1 KiB of chunks 64 j .. 64 j + 63
// (lane l takes chunk 64 j + l); R need not be a power of two (a 384-wide
// k-row is 48 chunks).  The MFMA fragments are then read with the transposing
// LDS read (ds_read_b64_tr_b16, see tr_frag); the swizzle spreads the four
// k-rows one 16-lane group of that read touches over distinct banks (an XOR
// by at most 12 keeps a chunk inside its 16-chunk group, so inside the row).
// Columns past the operand carry kOob from the start; k-rows past K are
// masked on a segment's last step only.
template <int R, int NW>
struct CopyNC {
  static constexpr int kRowB = R * 2;        // bytes of one k-row
  static constexpr int kLPR = kRowB / 16;    // 16-byte chunks per k-row
  static constexpr int kInstr = kBK * kLPR / 64 / NW;
  static_assert(kLPR >= 16 && kLPR % 16 == 0 && (kBK * kLPR) % (64 * NW) == 0,
                "k-rows must split evenly over the waves");
  Rsrc rs;
  const uint16_t* base;    // column row0, k = 0
  int64_t ld;
  int kt_base;             // step the descriptor starts at
  int kt_span;             // steps one descriptor covers with a 31-bit scalar offset
  uint32_t off[kInstr];    // k-row * ld * 2 + logical chunk * 16, or kOob
  __device__ __forceinline__ static int chunk_of(int i, int wave, int lane) {
    return (wave + i * NW) * 64 + lane;
  }
  __device__ __forceinline__ static int krow_of(int i, int wave, int lane) {
    return chunk_of(i, wave, lane) / kLPR;
  }
  __device__ __forceinline__ void prepare(const uint16_t* p, int64_t ldv, int row0, int nrows,
                                          int K, int wave, int lane, int) {
    base = p + row0;
    ld = ldv;
    kt_base = 0;
    kt_span = (int)((int64_t)0x40000000 / (ldv * 2 * kBK));   // >= 2: ld < 2^22
    rs = make_rsrc(base, (int64_t)K * ldv * 2);
#pragma unroll
    for (int i = 0; i < kInstr; ++i) {
      const int c = chunk_of(i, wave, lane);
      const int kr = c / kLPR;
      const int lc = (c - kr * kLPR) ^ (4 * (kr & 3));
      off[i] = row0 + lc * 8 < nrows ? (uint32_t)kr * (uint32_t)(ldv * 2) + (uint32_t)lc * 16u
                                     : kOob;
    }
  }
  template <bool TAIL>
  __device__ __forceinline__ void issue(uint8_t* lds_tile, int kt, int K, int wave, int lane,
                                        int) {
    if (kt - kt_base >= kt_span) {   // keep the scalar offset below 2^30
      kt_base = kt;
      rs = make_rsrc(base + (int64_t)kt * kBK * ld, (int64_t)(K - kt * kBK) * ld * 2);
    }
    const int soff = (kt - kt_base) * kBK * (int)(ld * 2);   // < 2^30
#pragma unroll
    for (int i = 0; i < kInstr; ++i) {
      uint32_t o = off[i];
      if (TAIL && kt * kBK + krow_of(i, wave, lane) >= K) o = kOob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(lds_tile + (wave + i * NW) * 1024), 16,
          (int)o, soff, 0, 0);
    }
  }
  __device__ __forceinline__ void commit(uint8_t*, int) {}
};

// Byte offset, within a stage of CopyNC's layout (row_bytes per k-row), of the
// 8-byte piece this lane hands to ds_read_b64_tr_b16 for the 32-row block at
// blk_row0, 16-deep step 0, first k quad.  A 16-lane group g of that read
// gathers a 4 (k) x 16 (rows) block: lane 4j + q supplies k-row j, rows 4q..4q+3,
// and lane i receives row i at the four k.  Lanes 0-15 / 16-31 take rows
// 0-15 / 16-31 of the block at k 0-7, lanes 32-63 the same rows at k 8-15,
// which is the operand layout of v_mfma_f32_32x32x16_bf16.  Step kk and the
// second k quad add (16 kk + 4) * row_bytes; (k-row % 4) stays the lane's j.
__device__ __forceinline__ int tr_base(int blk_row0, int row_bytes, int lane) {
  const int g = lane >> 4, jq = lane & 15, j = jq >> 2, q = jq & 3;
  const int kr = 8 * (g >> 1) + j;
  const int c = blk_row0 + 16 * (g & 1) + 4 * q;   // first row (column element) of the piece
  const int pc = (c >> 3) ^ (4 * j);
  return kr * row_bytes + pc * 16 + ((c >> 2) & 1) * 8;
}
typedef short v4i16 __attribute__((ext_vector_type(4)));
// Fragment of 8 consecutive k (two transposing reads, k quads 0 and 1).
__device__ __forceinline__ bf16x8 tr_frag(const uint8_t* p, int row_bytes) {
  typedef __attribute__((address_space(3))) v4i16 lds_v4;
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(p));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(p + 4 * row_bytes));
  const v4i16 v8[2] = {lo, hi};
  return __builtin_bit_cast(bf16x8, v8);
}

// Build switch: 0 stages every M/N-contiguous operand through registers
// (the earlier path, kept so the two can be timed against each other).
#ifndef DORA_MC_DIRECT
#define DORA_MC_DIRECT 1
#endif

template <int R, int NT, bool KC>
struct CopyOp;
template <int R, int NT>
struct CopyOp<R, NT, true> : CopyKC<R, NT / 64> {
  static constexpr bool kRegs = false;
  static constexpr bool kTr = false;
};
// Transposed operands go straight to LDS (read back transposed) when the tile
// has at least 128 rows; narrower tiles stage them through registers.
template <int R, int NT, bool DIRECT = (DORA_MC_DIRECT && R >= 128)>
struct CopyOpMC;
template <int R, int NT>
struct CopyOpMC<R, NT, true> : CopyNC<R, NT / 64> {
  static constexpr bool kRegs = false;
  static constexpr bool kTr = true;
};
template <int R, int NT>
struct CopyOpMC<R, NT, false> : CopyMC<R, NT> {
  static constexpr bool kRegs = true;
  static constexpr bool kTr = false;
};
template <int R, int NT>
struct CopyOp<R, NT, false> : CopyOpMC<R, NT> {};

// Tile index -> (tile_m, tile_n), XCD-grouped.  The hardware deals workgroups
// to the 8 XCDs round robin; the index is remapped so that each XCD takes a
// contiguous run, and runs walk groups of tile-rows column by column, so an
// XCD's tiles form a block whose operand panels its L2 shares.  Groups are 8
// tile-rows (an ~8 x 8 block per XCD on large outputs); when every column of
// tiles fits in an XCD's run with a block no wider than tall (skinny outputs,
// such as the rank-r projections), a group is exactly one XCD's run, so each
// XCD reads every panel of its tile-rows once instead of spilling half a group
// onto the next XCD.  Returns tile_m in .x and tile_n in .y.
__device__ __forceinline__ int2 tile_coords(int tiles_m, int tiles_n) {
  int L = blockIdx.x;
  const int nwg = gridDim.x;
  int group = 8;
  if ((nwg & 7) == 0) {
    L = (L & 7) * (nwg >> 3) + (L >> 3);
    const int run = nwg >> 3;
    if (tiles_n * tiles_n <= run && run % tiles_n == 0) group = run / tiles_n;
  }
  const int per_group = group * tiles_n;
  const int g = L / per_group;
  const int first = g * group;
  const int gsz = min(tiles_m - first, group);
  const int rem = L - g * per_group;
  return make_int2(first + rem % gsz, rem / gsz);
}

// bf16 kernels: a 1-D grid of tiles x K splits.  After the same XCD remap the
// index is split-major, so an XCD's contiguous run covers one K split (or a
// few): the operand slice a split shares between its tiles (e.g. A's K range
// in x A^T) is then read by one XCD's L2 instead of by all of them.  Returns
// tile_m, tile_n and the split index.
__device__ __forceinline__ int3 tile_split_coords(int tiles_m, int tiles_n, int nsplit) {
  int L = blockIdx.x;
  const int nwg = gridDim.x;
  const int tiles = tiles_m * tiles_n;
  int group = 8;
  if ((nwg & 7) == 0) {
    L = (L & 7) * (nwg >> 3) + (L >> 3);
    const int run = nwg >> 3;
    if (tiles_n * tiles_n <= run && run % tiles_n == 0) group = run / tiles_n;
  }
  const int split = L / tiles;
  L -= split * tiles;
  const int per_group = group * tiles_n;
  const int g = L / per_group;
  const int first = g * group;
  const int gsz = min(tiles_m - first, group);
  const int rem = L - g * per_group;
  (void)nsplit;
  return make_int3(first + rem % gsz, rem / gsz, split);
}

template <bool OUT_F32>
__device__ __forceinline__ void store4(void* cbase, int64_t ldc, int m, int n, float v0, float v1,
                                       float v2, float v3) {
  if (OUT_F32) {
    float* c = reinterpret_cast<float*>(cbase) + (int64_t)m * ldc + n;
    *reinterpret_cast<f32x4*>(c) = f32x4{v0, v1, v2, v3};
  } else {
    uint16_t* c = reinterpret_cast<uint16_t*>(cbase) + (int64_t)m * ldc + n;
    *reinterpret_cast<u32x2*>(c) = u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
  }
}

// g - 1 for output columns n..n+3 (compose epilogue).
template <bool BF>
__device__ __forceinline__ f32x4 gm1_4(const void* mag, const float* norm, int n) {
  f32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float mv = BF ? bf16_to_f32(reinterpret_cast<const uint16_t*>(mag)[n + e])
                        : reinterpret_cast<const float*>(mag)[n + e];
    const float nv = fmaxf(norm[n + e], kNormEps);
    r[e] = (mv - nv) / nv;
  }
  return r;
}

// g for output row m (merge epilogue).
template <bool BF>
__device__ __forceinline__ float g_row(const void* mag, const float* norm, int m) {
  const float mv = BF ? bf16_to_f32(reinterpret_cast<const uint16_t*>(mag)[m])
                      : reinterpret_cast<const float*>(mag)[m];
  return mv / fmaxf(norm[m], kNormEps);
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// s_waitcnt vmcnt(N) with the other counters left open (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Epilogue shared by the bf16 kernels: scale (and compose), then store.  bf16
// outputs are staged through LDS, one 32-row block of the wave's tile at a
// time in a region of its own (`stg`, 32 x (TN + 8) elements), so that every
// store is a whole 16-byte piece of a row; float32 outputs (split-K partials)
// go straight out.
template <int BM, int BN, int WM, int WN, int EPI, bool OUT_F32>
__device__ __forceinline__ void gemm_epilogue(f32x16 (&acc)[BM / WM / 32][BN / WN / 32],
                                              uint16_t* stg, int split, void* c, int64_t ldc,
                                              int64_t split_stride, float alpha, const void* mag,
                                              const float* nrm, const void* add, int64_t ld_add,
                                              int M, int N, int m0, int n0, int wave, int wm,
                                              int wn, int lane) {
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int MB = TM / 32, NB = TN / 32;
  constexpr int kStageLd = TN + 8;
  // Epilogue.  acc[i][j][v]: m = m0 + wm*TM + i*32 + lane%32,
  //                          n = n0 + wn*TN + j*32 + (v/4)*8 + (lane/32)*4 + v%4.
  void* cbase = OUT_F32 ? (void*)(reinterpret_cast<float*>(c) + split * split_stride)
                        : (void*)(reinterpret_cast<uint16_t*>(c) + split * split_stride);
  if constexpr (!OUT_F32) {
    // The K loop ended on a barrier, so every stage is free.  A wave's LDS
    // accesses complete in order, so block i + 1 may overwrite what block i
    // read back without a wait.
    f32x4 gm1[NB][4];   // compose: g - 1 of the lane's columns
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * TN + j * 32 + g * 8 + (lane >> 5) * 4;
        gm1[j][g] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (EPI == kEpiCompose && n < N) gm1[j][g] = gm1_4<true>(mag, nrm, n);
      }
    constexpr int kChunksPerRow = TN / 8;
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int mrow = m0 + wm * TM + i * 32;
      const int m = mrow + (lane & 31);
      const float grow = (EPI == kEpiMerge && m < M) ? g_row<true>(mag, nrm, m) : 0.f;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int nl = j * 32 + g * 8 + (lane >> 5) * 4;
          const int n = n0 + wn * TN + nl;
          u32x2 w = u32x2{0u, 0u};   // merge: the addend's four values at (m, n..n+3)
          if (EPI == kEpiMerge && m < M && n < N)
            w = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(add) +
                                                (int64_t)m * ld_add + n);
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float z = alpha * acc[i][j][g * 4 + e];
            if (EPI == kEpiMerge) {
              const uint32_t wv = w[e >> 1];
              v[e] = grow * ((e & 1 ? bf_hi(wv) : bf_lo(wv)) + z);
            } else {
              v[e] = (EPI == kEpiCompose) ? z + gm1[j][g][e] * z : z;
            }
          }
          *reinterpret_cast<u32x2*>(stg + (lane & 31) * kStageLd + nl) =
              u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        }
      }
#pragma unroll
      for (int c = lane; c < 32 * kChunksPerRow; c += 64) {
        const int row = c / kChunksPerRow, ch = c - row * kChunksPerRow;
        const int mm = mrow + row, n = n0 + wn * TN + ch * 8;
        const u32x4 val = *reinterpret_cast<const u32x4*>(stg + row * kStageLd + ch * 8);
        if (mm < M && n < N)
          *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(cbase) + (int64_t)mm * ldc + n) =
              val;
      }
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < NB; ++j) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int n = n0 + wn * TN + j * 32 + g * 8 + (lane >> 5) * 4;
      if (n >= N) continue;
      f32x4 gm1 = {0.f, 0.f, 0.f, 0.f};
      if (EPI == kEpiCompose) gm1 = gm1_4<!OUT_F32>(mag, nrm, n);
      static_assert(EPI != kEpiMerge || !OUT_F32, "merge writes the layer dtype");
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const int m = m0 + wm * TM + i * 32 + (lane & 31);
        if (m >= M) continue;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float z = alpha * acc[i][j][g * 4 + e];
          v[e] = (EPI == kEpiCompose) ? z + gm1[e] * z : z;
        }
        store4<OUT_F32>(cbase, ldc, m, n, v[0], v[1], v[2], v[3]);
      }
    }
  }
}

// s_barrier with no memory fence: the waits it needs are explicit.  The asm
// memory clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void barrier_nofence() { asm volatile("s_barrier" ::: "memory"); }

// Row-norm partials of the projection: atomic (write-through) stores when the
// kernel finishes the norms itself and another workgroup reads them, plain
// stores otherwise; and the matching agent-scope load.
__device__ __forceinline__ void put_partial(float* dst, float v, const float* finishing) {
  if (finishing)
    __hip_atomic_store(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *dst = v;
}
__device__ __forceinline__ float get_partial(const float* src) {
  return __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// NSEG: the most K segments the kernel walks (2, or 3 for the norm's projection
// and the undetached-gradient products): every segment's pointers, strides
// and bounds live in scalar registers, which the largest tiles have to spare.
template <int BM, int BN, int WM, int WN, bool AKC, bool BKC, int EPI, bool OUT_F32, int NSEG,
          int S>
__global__ __launch_bounds__(WM * WN * 64) void dora_gemm_bf16(const KArgs p) {
  static_assert(NSEG == 2 || NSEG == 3, "two or three K segments");
  static_assert(S >= 2 && S <= 4, "two to four stages");
  constexpr int NT = WM * WN * 64, NW = WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int MB = TM / 32, NB = TN / 32;
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be a multiple of 32");
  using CA = CopyOp<BM, NT, AKC>;
  using CB = CopyOp<BN, NT, BKC>;
  constexpr bool kRegs = CA::kRegs || CB::kRegs;
  static_assert(S == 2 || !kRegs, "register-staged copies take the two-stage pipeline");
  constexpr bool kTrA = CA::kTr, kTrB = CB::kTr;
  // LDS.  With an operand read by the transposing read, or more than two
  // stages, one object per operand and stage: kept apart, they let the compiler
  // see that a stage's fragment reads cannot touch the other stages, which the
  // copies in flight are filling (without that it waits for every copy before
  // a transposing read).  Otherwise one object [A stage 0 | A stage 1 | B
  // stage 0 | B stage 1], so that every fragment read is a per-lane base plus
  // an immediate offset.
  constexpr bool kSplit = kTrA || kTrB || S > 2;
  constexpr int ABYTES = BM * kRowBytes, BBYTES = BN * kRowBytes;
  constexpr int BBASE = kSplit ? 0 : 2 * ABYTES;   // B's offset within its object
  static_assert(kSplit || (ABYTES + (MB > 2 ? 64 * kRowBytes : 0) < 65536 &&
                           BBYTES + (NB > 2 ? 64 * kRowBytes : 0) < 65536),
                "stage offsets must fit the LDS immediate");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kSplit ? ABYTES : 2 * (ABYTES + BBYTES)];
  __shared__ __attribute__((aligned(1024))) uint8_t sA1[kSplit ? ABYTES : 1];
  __shared__ __attribute__((aligned(1024))) uint8_t sB0[kSplit ? BBYTES : 1];
  __shared__ __attribute__((aligned(1024))) uint8_t sB1[kSplit ? BBYTES : 1];
  __shared__ __attribute__((aligned(1024))) uint8_t sA2[S > 2 ? ABYTES : 1];
  __shared__ __attribute__((aligned(1024))) uint8_t sB2[S > 2 ? BBYTES : 1];
  __shared__ __attribute__((aligned(1024))) uint8_t sA3[S > 3 ? ABYTES : 1];
  __shared__ __attribute__((aligned(1024))) uint8_t sB3[S > 3 ? BBYTES : 1];
  static_assert(S * (ABYTES + BBYTES) <= 160 * 1024, "stages must fit the LDS");
  // bf16 epilogue: each wave stages 32 rows of its tile at a time in a region
  // of its own.
  constexpr int kStageLd = TN + 8;
  constexpr int kStgBytes = 32 * kStageLd * 2;
  static_assert(OUT_F32 || (kSplit ? ((NW + 3) / 4) * kStgBytes <= (ABYTES < BBYTES ? ABYTES : BBYTES)
                                   : NW * kStgBytes <= 2 * (ABYTES + BBYTES)),
                "epilogue staging must fit the stage objects");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % WM, wn = wave / WM;
  const int M = p.M, N = p.N;
  const int3 tc = tile_split_coords(p.tiles_m, p.tiles_n, p.nsplit);
  const int m0 = __builtin_amdgcn_readfirstlane(tc.x * BM);
  const int n0 = __builtin_amdgcn_readfirstlane(tc.y * BN);
  const int split = __builtin_amdgcn_readfirstlane(tc.z);
  const int kt_lo = split * p.kt_per_split;
  const int kt_hi = min(kt_lo + p.kt_per_split, p.kt_total);
  constexpr bool k3 = NSEG == 3;
  const int kt_end0 = p.kt_end[0], kt_end1 = p.kt_end[1], kt_end2 = k3 ? p.kt_end[2] : 0;
  const uint16_t *a0 = p.a[0], *a1 = p.a[1], *a2 = k3 ? p.a[2] : nullptr;
  const uint16_t *b0 = p.b[0], *b1 = p.b[1], *b2 = k3 ? p.b[2] : nullptr;
  const int64_t lda0 = p.lda[0], lda1 = p.lda[1], lda2 = k3 ? p.lda[2] : 0;
  const int64_t ldb0 = p.ldb[0], ldb1 = p.ldb[1], ldb2 = k3 ? p.ldb[2] : 0;
  const int K0 = p.K[0], K1 = p.K[1], K2 = k3 ? p.K[2] : 0;

  f32x16 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  constexpr bool kRowSq = EPI == kEpiNorm;
  // kEpiNorm: the waves of the first wave column of the first column tile sum
  // the squares of the opA fragments they read (VALU work beside the MFMAs) and
  // keep the sums of segment 0.
  float sq[2][MB];   // kEpiNorm: per-lane partial sums of squares of the lane's opA rows
  float sq0[MB];     // the same at the end of segment 0
#pragma unroll
  for (int i = 0; i < MB; ++i) sq[0][i] = sq[1][i] = sq0[i] = 0.f;

  // Fragment read bases: the swizzle of row wm*TM + i*32 + lane%32 depends on i
  // only through its parity, and the chunk of step kk only through an XOR.
  uint32_t ra[2][4], rb[2][4];
#pragma unroll
  for (int par = 0; par < 2; ++par)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int rowa = wm * TM + par * 32 + (lane & 31);
      const int rowb = wn * TN + par * 32 + (lane & 31);
      const int ch = kk * 2 + (lane >> 5);
      ra[par][kk] = (uint32_t)(rowa * kRowBytes + ((ch ^ swz(rowa)) << 4));
      rb[par][kk] = (uint32_t)(BBASE + rowb * kRowBytes + ((ch ^ swz(rowb)) << 4));
    }
  // Operands kept k-major in LDS are read with the transposing read: one base
  // per 32-row block (the chunk swizzle mixes the block index with the k-row).
  static_assert(52 * BM * 2 < 65536 && 52 * BN * 2 < 65536,
                "transposing-read offsets must fit the LDS immediate");
  uint32_t ta[kTrA ? MB : 1], tb[kTrB ? NB : 1];
  if constexpr (kTrA) {
#pragma unroll
    for (int i = 0; i < MB; ++i) ta[i] = (uint32_t)tr_base(wm * TM + i * 32, BM * 2, lane);
  }
  if constexpr (kTrB) {
#pragma unroll
    for (int j = 0; j < NB; ++j) tb[j] = (uint32_t)tr_base(wn * TN + j * 32, BN * 2, lane);
  }

  // Stage SB of each operand (B's offset BBASE within the object is in the
  // fragment bases and added for the copies).
#define DORA_A(SB) \
  (kSplit ? ((SB) == 0 ? smem : (SB) == 1 ? sA1 : (SB) == 2 ? sA2 : sA3) : smem + (SB) * ABYTES)
#define DORA_B(SB) \
  (kSplit ? ((SB) == 0 ? sB0 : (SB) == 1 ? sB1 : (SB) == 2 ? sB2 : sB3) : smem + (SB) * BBYTES)
  // Copies of segment step KR into stage SB.
#define DORA_FETCH(KR, SB)                                                                 \
  do {                                                                                     \
    uint8_t* sa_ = DORA_A(SB);                                                             \
    uint8_t* sb_ = DORA_B(SB) + BBASE;                                                     \
    if (partial && (KR) == last) {                                                         \
      ca.template issue<true>(sa_, (KR), Ks, wave, lane, tid);                             \
      cb.template issue<true>(sb_, (KR), Ks, wave, lane, tid);                             \
    } else {                                                                               \
      ca.template issue<false>(sa_, (KR), Ks, wave, lane, tid);                            \
      cb.template issue<false>(sb_, (KR), Ks, wave, lane, tid);                            \
    }                                                                                      \
  } while (0)
  // Register-staged copies of stage SB land in LDS (after their loads).
#define DORA_COMMIT(SB)                                                                    \
  do {                                                                                     \
    if (kRegs) {                                                                           \
      wait_vmem();                                                                         \
      ca.commit(DORA_A(SB), tid);                                                          \
      cb.commit(DORA_B(SB) + BBASE, tid);                                                  \
    }                                                                                      \
  } while (0)

  bf16x8 af[2][MB], bfr[2][NB];
#define DORA_READ(SET, SB, KK)                                                             \
  do {                                                                                     \
    if constexpr (kTrA) {                                                                  \
      _Pragma("unroll") for (int i = 0; i < MB; ++i) af[SET][i] =                          \
          tr_frag(DORA_A(SB) + ta[i] + (KK) * 16 * BM * 2, BM * 2);                        \
    } else {                                                                               \
      _Pragma("unroll") for (int i = 0; i < MB; ++i) af[SET][i] =                          \
          *reinterpret_cast<const bf16x8*>(DORA_A(SB) + ra[i & 1][KK] +                    \
                                           (i >> 1) * 64 * kRowBytes);                     \
    }                                                                                      \
    if constexpr (kTrB) {                                                                  \
      _Pragma("unroll") for (int j = 0; j < NB; ++j) bfr[SET][j] =                         \
          tr_frag(DORA_B(SB) + tb[j] + (KK) * 16 * BN * 2, BN * 2);                        \
    } else {                                                                               \
      _Pragma("unroll") for (int j = 0; j < NB; ++j) bfr[SET][j] =                         \
          *reinterpret_cast<const bf16x8*>(DORA_B(SB) + rb[j & 1][KK] +                    \
                                           (j >> 1) * 64 * kRowBytes);                     \
    }                                                                                      \
  } while (0)
  // One stage: four 16-deep steps, fragments of step kk+1 read during step kk.
#define DORA_MMA(SB, SQ)                                                                   \
  do {                                                                                     \
    DORA_READ(0, SB, 0);                                                                   \
    _Pragma("unroll") for (int kk = 0; kk < 4; ++kk) {                                     \
      if (kk < 3) {                                                                        \
        if (kk & 1) DORA_READ(0, SB, kk + 1);                                              \
        else DORA_READ(1, SB, kk + 1);                                                     \
      }                                                                                    \
      __builtin_amdgcn_sched_barrier(0);                                                   \
      _Pragma("unroll") for (int i = 0; i < MB; ++i)                                       \
          _Pragma("unroll") for (int j = 0; j < NB; ++j) acc[i][j] =                       \
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[kk & 1][j], af[kk & 1][i],      \
                                                      acc[i][j], 0, 0, 0);                 \
      __builtin_amdgcn_sched_barrier(0);                                                   \
      if (SQ) {                                                                            \
        /* elements 2q, 2q+1 share one 32-bit register: a shuffle of that pair */          \
        /* selects it without repacking                                        */          \
        _Pragma("unroll") for (int i = 0; i < MB; ++i) {                                   \
          const bf16x8 f_ = af[kk & 1][i];                                                 \
          const bf16x2 h0_ = __builtin_shufflevector(f_, f_, 0, 1);                        \
          const bf16x2 h1_ = __builtin_shufflevector(f_, f_, 2, 3);                        \
          const bf16x2 h2_ = __builtin_shufflevector(f_, f_, 4, 5);                        \
          const bf16x2 h3_ = __builtin_shufflevector(f_, f_, 6, 7);                        \
          float t_ = sq[kk & 1][i];                                                        \
          t_ = __builtin_amdgcn_fdot2_f32_bf16(h0_, h0_, t_, false);                       \
          t_ = __builtin_amdgcn_fdot2_f32_bf16(h1_, h1_, t_, false);                       \
          t_ = __builtin_amdgcn_fdot2_f32_bf16(h2_, h2_, t_, false);                       \
          t_ = __builtin_amdgcn_fdot2_f32_bf16(h3_, h3_, t_, false);                       \
          sq[kk & 1][i] = t_;                                                              \
        }                                                                                  \
      }                                                                                    \
    }                                                                                      \
  } while (0)

  // Segments one after the other; the pipeline restarts at each (at most two
  // restarts per launch), so within a segment the copy state is loop-invariant.
#pragma unroll 1
  for (int seg = 0; seg < NSEG; ++seg) {
    const int s_lo = seg == 0 ? 0 : (seg == 1 ? kt_end0 : kt_end1);
    const int s_hi = seg == 0 ? kt_end0 : (seg == 1 ? kt_end1 : kt_end2);
    const int lo = max(kt_lo, s_lo), hi = min(kt_hi, s_hi);
    if (lo >= hi) continue;
    const int Ks = seg == 0 ? K0 : (seg == 1 ? K1 : K2);
    const bool partial = (Ks % kBK) != 0;
    const int last = s_hi - 1 - s_lo;   // the segment's last step
    CA ca;
    CB cb;
    ca.prepare(seg == 0 ? a0 : (seg == 1 ? a1 : a2), seg == 0 ? lda0 : (seg == 1 ? lda1 : lda2),
               m0, M, Ks, wave, lane, tid);
    cb.prepare(seg == 0 ? b0 : (seg == 1 ? b1 : b2), seg == 0 ? ldb0 : (seg == 1 ? ldb1 : ldb2),
               n0, N, Ks, wave, lane, tid);
    const int r_lo = lo - s_lo, r_hi = hi - s_lo;
    // Two stages: the copies of step kr + 1 fly while step kr is multiplied.
#define DORA_STAGES(SQ)                                                                    \
  for (int kr = r_lo; kr < r_hi; kr += 2) {                                                \
    if (kr + 1 < r_hi) DORA_FETCH(kr + 1, 1);                                              \
    DORA_MMA(0, SQ);                                                                       \
    if (kr + 1 < r_hi) DORA_COMMIT(1);                                                     \
    wait_vmem();                                                                           \
    barrier_nofence();                                                                     \
    if (kr + 1 >= r_hi) break;                                                             \
    if (kr + 2 < r_hi) DORA_FETCH(kr + 2, 0);                                              \
    DORA_MMA(1, SQ);                                                                       \
    if (kr + 2 < r_hi) DORA_COMMIT(0);                                                     \
    wait_vmem();                                                                           \
    barrier_nofence();                                                                     \
  }
    // Row sums of squares ride on the fragments that the first wave column of
    // the first column tile already holds (a flag fixed for the whole kernel,
    // so the compiler keeps the other waves' loop free of it); the sums of
    // segment 0 are kept when it ends.
    const bool sq_w = kRowSq && wn == 0 && tc.y == 0;
    if constexpr (S == 2) {
      DORA_FETCH(r_lo, 0);
      DORA_COMMIT(0);
      wait_vmem();
      barrier_nofence();
      DORA_STAGES(sq_w)
    } else {
      // A ring of S stages: the copies of the next S - 1 steps fly while a step
      // is multiplied.  Step q lives in slot (q - r_lo) % S; it has landed once
      // at most the copies of the steps issued after it are outstanding (vmcnt
      // retires loads in order), and the barrier after that wait also tells
      // that every wave is done with slot (q - 1) % S, which then takes step
      // q + S - 1.
      constexpr int kPS = CA::kInstr + CB::kInstr;   // copy instructions per step and wave
#pragma unroll
      for (int j = 0; j < S - 1; ++j)
        if (r_lo + j < r_hi) DORA_FETCH(r_lo + j, j);
      for (int kr = r_lo; kr < r_hi; kr += S) {
#pragma unroll
        for (int J = 0; J < S; ++J) {
          const int q = kr + J;
          if (q >= r_hi) break;
          const int later = min(S - 2, r_hi - 1 - q);
          if (S > 3 && later >= 2) wait_vmem_le<(S > 3 ? 2 * kPS : 0)>();
          else if (later >= 1) wait_vmem_le<kPS>();
          else wait_vmem_le<0>();
          barrier_nofence();
          if (q + S - 1 < r_hi) DORA_FETCH(q + S - 1, (J + S - 1) % S);
          DORA_MMA(J, sq_w);
        }
      }
      barrier_nofence();   // every slot read before the next segment or the epilogue reuses LDS
    }
    if (kRowSq && seg == 0) {
#pragma unroll
      for (int i = 0; i < MB; ++i) sq0[i] = sq[0][i] + sq[1][i];
    }
  }
#undef DORA_STAGES
#undef DORA_FETCH
#undef DORA_COMMIT
#undef DORA_READ
#undef DORA_MMA
#undef DORA_A
#undef DORA_B

  if constexpr (kRowSq) {
    // Lane l and lane l + 32 hold the two halves of every 16-deep step of
    // one row; each split writes its partial (zero if it saw no segment-0 step).
    if (wn == 0 && tc.y == 0) {
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        float v = sq0[i];
        v += __shfl_xor(v, 32);
        const int m = m0 + wm * TM + i * 32 + lane;
        if (lane < 32 && m < M) put_partial(p.rowsq + (int64_t)split * M + m, v, p.norm_out);
      }
    }
    const int64_t slot = (int64_t)split * p.tiles_n + tc.y;
    // C itself is not stored: each lane dots its accumulators with the rows
    // of `add` at the same (m, n) (in-lane over j, g, e, then the two lanes
    // that share a row), one partial per split, column tile and wave column.
    const uint16_t* addp = reinterpret_cast<const uint16_t*>(p.add);
    float dot[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) dot[i] = 0.f;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * TN + j * 32 + g * 8 + (lane >> 5) * 4;
        if (n >= N) continue;   // N % 4 == 0: n < N covers n..n+3
#pragma unroll
        for (int i = 0; i < MB; ++i) {
          const int m = m0 + wm * TM + i * 32 + (lane & 31);
          if (m >= M) continue;
          const u32x2 w = *reinterpret_cast<const u32x2*>(addp + (int64_t)m * p.ld_add + n);
          dot[i] = fmaf(bf_lo(w[0]), acc[i][j][g * 4 + 0], dot[i]);
          dot[i] = fmaf(bf_hi(w[0]), acc[i][j][g * 4 + 1], dot[i]);
          dot[i] = fmaf(bf_lo(w[1]), acc[i][j][g * 4 + 2], dot[i]);
          dot[i] = fmaf(bf_hi(w[1]), acc[i][j][g * 4 + 3], dot[i]);
        }
      }
    }
    // The WN wave columns hold partial dots of the same rows: they meet in LDS
    // (free after the K loop's final barrier) and the first wave column adds
    // them in wave-column order, one partial per split and column tile.
    float* red = reinterpret_cast<float*>(smem);   // [WN][BM]
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      float v = dot[i];
      v += __shfl_xor(v, 32);
      if (lane < 32) red[wn * BM + wm * TM + i * 32 + lane] = v;
    }
    __syncthreads();
    if (wn == 0) {
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const int rr = wm * TM + i * 32 + lane;
        const int m = m0 + rr;
        float v = red[rr];
#pragma unroll
        for (int w = 1; w < WN; ++w) v += red[w * BM + rr];
        if (lane < 32 && m < M) put_partial(p.rowdot + slot * M + m, p.alpha * v, p.norm_out);
      }
    }
    if (p.norm_out) {
      // The last workgroup of this tile row to finish (over K splits and
      // column tiles) adds every partial of its rows in a fixed order:
      // n_m = sqrt(max(0, sum_z rowsq[z][m] + sum_q rowdot[q][m])).  The
      // partials travel as agent-scope atomic stores and loads, which write
      // through and read past the per-XCD L2s; each workgroup waits for its
      // stores to complete before it counts itself.  (Agent-scope fences would
      // write back and invalidate the whole L2 instead, evicting the operand
      // panels the other workgroups are still reading.)
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      int* last = reinterpret_cast<int*>(smem) + WN * BM;   // past `red`, which is done
      if (tid == 0) {
        const uint32_t before = __hip_atomic_fetch_add(p.done + tc.x, 1u, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT);
        *last = before + 1 == (uint32_t)(p.nsplit * p.tiles_n);
      }
      __syncthreads();
      if (*last) {
        // Four lanes per row, each adding a contiguous quarter of the row's
        // partials [rowsq z = 0..S-1, then rowdot q = 0..Q-1] with all of its
        // loads in flight together; the quarters are then added in order.
        const int nsq = p.nsplit, L = nsq + p.nsplit * p.tiles_n;
        const int chunk = (L + 3) / 4, quarter = tid & 3;
        const int j0 = quarter * chunk, j1 = min(L, j0 + chunk);
        for (int rr = tid >> 2; rr < BM; rr += NT / 4) {   // whole 4-lane groups stay together
          const int m = m0 + rr;
          float part = 0.f;
          if (m < M) {
            for (int jb = j0; jb < j1; jb += 8) {
              float v[8];
#pragma unroll
              for (int u = 0; u < 8; ++u) {
                const int j = jb + u;
                v[u] = j >= j1 ? 0.f
                       : get_partial(j < nsq ? p.rowsq + (int64_t)j * M + m
                                             : p.rowdot + (int64_t)(j - nsq) * M + m);
              }
#pragma unroll
              for (int u = 0; u < 8; ++u) part += v[u];
            }
          }
          const int base_lane = lane & ~3;
          const float q0 = __shfl(part, base_lane), q1 = __shfl(part, base_lane + 1);
          const float q2 = __shfl(part, base_lane + 2), q3 = __shfl(part, base_lane + 3);
          if (quarter == 0 && m < M) p.norm_out[m] = sqrtf(fmaxf(((q0 + q1) + q2) + q3, 0.f));
        }
      }
    }
    return;
  }

  uint8_t* const stg_obj =
      !kSplit ? smem + wave * kStgBytes
              : ((wave & 3) == 0 ? smem : (wave & 3) == 1 ? sA1 : (wave & 3) == 2 ? sB0 : sB1) +
                    (wave >> 2) * kStgBytes;
  uint16_t* const stg = reinterpret_cast<uint16_t*>(stg_obj);
  gemm_epilogue<BM, BN, WM, WN, EPI, OUT_F32>(acc, stg, split, p.c, p.ldc, p.split_stride, p.alpha, p.mag,
                                                p.norm, p.add, p.ld_add, M, N, m0, n0, wave, wm,
                                                wn, lane);
}

// float32 layers: 64x64 tiles on the fp32 matrix cores (v_mfma_f32_32x32x2_f32),
// one 32x32 block per wave.  A 64-deep K step is staged through registers into
// k-major LDS tiles (every load of the step in flight before the first LDS
// store, so a step costs one memory latency); step pair (2j, 2j+1) is one
// MFMA whose lanes 0-31 take k = 2j and lanes 32-63 k = 2j + 1 of their row.
// As in the bf16 kernels the MFMA is issued as opB-block x opA-block^T, so each
// lane ends up holding four consecutive output columns of one output row.
template <bool AKC, bool BKC, int EPI>
__global__ __launch_bounds__(256) void dora_gemm_f32(const KArgs p) {
  constexpr int BM = 64, BN = 64, BKF = kBK;   // one 64-deep step per pass through LDS
  constexpr int kPer = BM * BKF / 256;          // elements of each operand per thread and pass
  __shared__ float As[BKF][BM + 4];
  __shared__ float Bs[BKF][BN + 4];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;      // the wave's 32x32 block of the tile
  const int2 tc = tile_coords(p.tiles_m, p.tiles_n);
  const int m0 = tc.x * BM, n0 = tc.y * BN;
  f32x16 acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
  const int kt_total = p.kt_total;   // in 64-deep units, shared with the bf16 path
  const int kt_lo = blockIdx.y * p.kt_per_split;
  const int kt_hi = min(kt_lo + p.kt_per_split, kt_total);
  const int ra = wm * 32 + (lane & 31), rb = wn * 32 + (lane & 31), kh = lane >> 5;
  for (int kt = kt_lo; kt < kt_hi; ++kt) {
    const int s = kt < p.kt_end[0] ? 0 : (kt < p.kt_end[1] ? 1 : 2);
    const int k0 = (kt - (s == 0 ? 0 : (s == 1 ? p.kt_end[0] : p.kt_end[1]))) * kBK;
    const float* a = reinterpret_cast<const float*>(s == 0 ? p.a[0] : (s == 1 ? p.a[1] : p.a[2]));
    const float* b = reinterpret_cast<const float*>(s == 0 ? p.b[0] : (s == 1 ? p.b[1] : p.b[2]));
    const int64_t lda = s == 0 ? p.lda[0] : (s == 1 ? p.lda[1] : p.lda[2]);
    const int64_t ldb = s == 0 ? p.ldb[0] : (s == 1 ? p.ldb[1] : p.ldb[2]);
    const int Ks = s == 0 ? p.K[0] : (s == 1 ? p.K[1] : p.K[2]);
    // Element e of a K-contiguous operand is (row e / 64, k e % 64): 64 lanes
    // read one row's 256 contiguous bytes.
    float va[kPer], vb[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = tid + i * 256;
      const int mm = AKC ? e / BKF : e % BM, kk = AKC ? e % BKF : e / BM;
      const int gm = m0 + mm, gk = k0 + kk;
      va[i] = (gm < p.M && gk < Ks) ? (AKC ? a[(int64_t)gm * lda + gk] : a[(int64_t)gk * lda + gm])
                                    : 0.f;
      const int nn = BKC ? e / BKF : e % BN, kb = BKC ? e % BKF : e / BN;
      const int gn = n0 + nn, gk2 = k0 + kb;
      vb[i] = (gn < p.N && gk2 < Ks) ? (BKC ? b[(int64_t)gn * ldb + gk2] : b[(int64_t)gk2 * ldb + gn])
                                     : 0.f;
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = tid + i * 256;
      const int mm = AKC ? e / BKF : e % BM, kk = AKC ? e % BKF : e / BM;
      As[kk][mm] = va[i];
      const int nn = BKC ? e / BKF : e % BN, kb = BKC ? e % BKF : e / BN;
      Bs[kb][nn] = vb[i];
    }
    __syncthreads();
#pragma unroll 8
    for (int j = 0; j < BKF / 2; ++j)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(Bs[2 * j + kh][rb], As[2 * j + kh][ra], acc, 0, 0, 0);
    __syncthreads();
  }
  // acc[v]: row m = m0 + wm*32 + lane%32, column n = n0 + wn*32 + (v/4)*8 + (lane/32)*4 + v%4
  float* c = reinterpret_cast<float*>(p.c) + blockIdx.y * p.split_stride;
  const int m = m0 + ra;
  if (m >= p.M) return;
  float gr = 0.f;
  if (EPI == kEpiMerge) gr = g_row<false>(p.mag, p.norm, m);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int n = n0 + wn * 32 + g * 8 + kh * 4;
    if (n >= p.N) continue;   // N % 4 == 0: n < N covers n..n+3
    f32x4 gm1 = {0.f, 0.f, 0.f, 0.f};
    if (EPI == kEpiCompose) gm1 = gm1_4<false>(p.mag, p.norm, n);
    f32x4 w = {0.f, 0.f, 0.f, 0.f};
    if (EPI == kEpiMerge)
      w = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(p.add) + (int64_t)m * p.ld_add + n);
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float z = p.alpha * acc[g * 4 + e];
      v[e] = (EPI == kEpiMerge) ? gr * (w[e] + z) : ((EPI == kEpiCompose) ? z + gm1[e] * z : z);
    }
    store4<true>(c, p.ldc, m, n, v[0], v[1], v[2], v[3]);
  }
}

// ---- split-K reduction ----------------------------------------------------------
// out[i] = alpha * sum_{z < S} part[z][i] over M*N elements, fixed order; with
// mag given, the compose epilogue is applied to the sum.
__global__ __launch_bounds__(256) void dora_splitk_reduce(const float* part, int S, int64_t n4,
                                                          int64_t stride, float alpha, void* out,
                                                          int out_bf16, const void* mag,
                                                          int mag_bf16, const float* nrm, int N) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  // partials added in index order, their loads issued four at a time
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int z0 = 0; z0 < S; z0 += 4) {
    f32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (z0 + u < S) v[u] = reinterpret_cast<const f32x4*>(part + (z0 + u) * stride)[i];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (z0 + u < S) acc = (z0 + u == 0) ? v[u] : acc + v[u];
  }
  acc *= alpha;
  if (mag) {   // compose epilogue: y = z + (g - 1) z per column, as the GEMM epilogue forms it
    const int n = (int)((i * 4) % N);
    const f32x4 gm1 = mag_bf16 ? gm1_4<true>(mag, nrm, n) : gm1_4<false>(mag, nrm, n);
    acc += gm1 * acc;
  }
  if (out_bf16)
    reinterpret_cast<u32x2*>(out)[i] = u32x2{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
  else
    reinterpret_cast<f32x4*>(out)[i] = acc;
}

// ---- host-side dispatch -----------------------------------------------------

// Tile configurations: BM x BN workgroup tile, WM x WN waves, pipeline stages.
struct Cfg {
  int bm, bn, wm, wn, st;
};
constexpr Cfg kCfgs[] = {
    {256, 256, 2, 4, 2},   // 0: 8 waves, 128x64 per wave
    {256, 128, 2, 2, 2},   // 1: 4 waves, 128x64 per wave
    {128, 128, 2, 2, 2},   // 2: 4 waves, 64x64 per wave
    {128, 256, 2, 2, 2},   // 3: 4 waves, 64x128 per wave
    {64, 64, 2, 2, 2},     // 4: 4 waves, 32x32 per wave
    {256, 128, 4, 2, 2},   // 5: 8 waves, 64x64 per wave
    {128, 384, 2, 4, 2},   // 6: 8 waves, 64x96 per wave (N = rank 384 in one tile)
    {384, 128, 4, 2, 2},   // 7: 8 waves, 96x64 per wave (M = rank 384 in one tile)
    {128, 192, 2, 2, 2},   // 8: 4 waves, 64x96 per wave (two workgroups per CU; K-contiguous only)
    {128, 128, 4, 2, 3},   // 9: 8 waves, 32x64 per wave, three stages (one workgroup per CU)
};
constexpr int kNumCfgs = sizeof(kCfgs) / sizeof(kCfgs[0]);

template <int BM, int BN, int WM, int WN, int S, bool AKC, bool BKC, int EPI, bool OUT_F32,
          int NSEG>
hipError_t launch_one(const KArgs& a, dim3 grid, hipStream_t st) {
  if (a.nseg > NSEG) return hipErrorInvalidValue;
  hipLaunchKernelGGL((dora_gemm_bf16<BM, BN, WM, WN, AKC, BKC, EPI, OUT_F32, NSEG, S>), grid,
                     dim3(WM * WN * 64), 0, st, a);
  return hipGetLastError();
}

// The store epilogues come with two or three segments, picked by the problem.
template <int BM, int BN, int WM, int WN, int S, bool AKC, bool BKC, bool OUT_F32>
hipError_t launch_store(const KArgs& a, dim3 grid, hipStream_t st) {
  if (a.nseg > 2)
    return launch_one<BM, BN, WM, WN, S, AKC, BKC, kEpiStore, OUT_F32, 3>(a, grid, st);
  return launch_one<BM, BN, WM, WN, S, AKC, BKC, kEpiStore, OUT_F32, 2>(a, grid, st);
}

template <int BM, int BN, int WM, int WN, int S, bool AKC, bool BKC>
hipError_t launch_bf16(const KArgs& a, int epi, bool out_f32, dim3 grid, hipStream_t st) {
  if (out_f32) {
    if constexpr (AKC && BKC) {   // the norm's projection: W0 and A are K-contiguous
      if (epi == kEpiNorm)
        return launch_one<BM, BN, WM, WN, S, AKC, BKC, kEpiNorm, true, 3>(a, grid, st);
    }
    if (epi == kEpiNorm) return hipErrorInvalidValue;
    return launch_store<BM, BN, WM, WN, S, AKC, BKC, true>(a, grid, st);
  }
  if constexpr (AKC && BKC) {   // the compose epilogue belongs to the forward (K-contiguous) GEMM
    if (epi == kEpiCompose)
      return launch_one<BM, BN, WM, WN, S, AKC, BKC, kEpiCompose, false, 2>(a, grid, st);
    if (epi != kEpiStore) return hipErrorInvalidValue;
  } else if constexpr (AKC && !BKC) {   // the merge epilogue belongs to B . A
    if (epi == kEpiMerge)
      return launch_one<BM, BN, WM, WN, S, AKC, BKC, kEpiMerge, false, 2>(a, grid, st);
    if (epi != kEpiStore) return hipErrorInvalidValue;
  } else {
    if (epi != kEpiStore) return hipErrorInvalidValue;
  }
  return launch_store<BM, BN, WM, WN, S, AKC, BKC, false>(a, grid, st);
}

// An M/N-contiguous operand is copied straight to LDS when its tile side is a
// multiple of 128 (whole 16-chunk groups per k-row) and through registers
// below 128 rows; other widths take K-contiguous operands only.
template <int R>
constexpr bool kMcOk = R % 128 == 0 || (R < 128 && R % 64 == 0);

template <int BM, int BN, int WM, int WN, int S>
hipError_t launch_layout(bool akc, bool bkc, const KArgs& a, int epi, bool out_f32, dim3 grid,
                         hipStream_t st) {
  if (akc && bkc) return launch_bf16<BM, BN, WM, WN, S, true, true>(a, epi, out_f32, grid, st);
  if constexpr (kMcOk<BN>) {
    if (akc && !bkc) return launch_bf16<BM, BN, WM, WN, S, true, false>(a, epi, out_f32, grid, st);
    // two register-staged operands do not fit beside a 256 x 256 tile's accumulators
    // (transposed operands of 128 rows or more are copied straight to LDS)
    if constexpr (kMcOk<BM> &&
                  (BM * BN <= 256 * 128 || (DORA_MC_DIRECT && BM >= 128 && BN >= 128)))
      if (!akc && !bkc) return launch_bf16<BM, BN, WM, WN, S, false, false>(a, epi, out_f32, grid, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_cfg(int cfg, bool akc, bool bkc, const KArgs& a, int epi, bool out_f32, dim3 grid,
                      hipStream_t st) {
  switch (cfg) {
    case 0: return launch_layout<256, 256, 2, 4, 2>(akc, bkc, a, epi, out_f32, grid, st);
    case 1: return launch_layout<256, 128, 2, 2, 2>(akc, bkc, a, epi, out_f32, grid, st);
    case 2: return launch_layout<128, 128, 2, 2, 2>(akc, bkc, a, epi, out_f32, grid, st);
    case 3: return launch_layout<128, 256, 2, 2, 2>(akc, bkc, a, epi, out_f32, grid, st);
    case 4: return launch_layout<64, 64, 2, 2, 2>(akc, bkc, a, epi, out_f32, grid, st);
    case 5: return launch_layout<256, 128, 4, 2, 2>(akc, bkc, a, epi, out_f32, grid, st);
    case 6: return launch_layout<128, 384, 2, 4, 2>(akc, bkc, a, epi, out_f32, grid, st);
    case 7: return launch_layout<384, 128, 4, 2, 2>(akc, bkc, a, epi, out_f32, grid, st);
    case 8: return launch_layout<128, 192, 2, 2, 2>(akc, bkc, a, epi, out_f32, grid, st);
    case 9: return launch_layout<128, 128, 4, 2, 3>(akc, bkc, a, epi, out_f32, grid, st);
    default: return hipErrorInvalidValue;
  }
}

template <bool AKC, bool BKC>
hipError_t launch_f32(const KArgs& a, int epi, dim3 grid, hipStream_t st) {
  if (epi == kEpiCompose)
    hipLaunchKernelGGL((dora_gemm_f32<AKC, BKC, kEpiCompose>), grid, dim3(256), 0, st, a);
  else if (epi == kEpiMerge && AKC && !BKC)
    hipLaunchKernelGGL((dora_gemm_f32<AKC, BKC, kEpiMerge>), grid, dim3(256), 0, st, a);
  else if (epi == kEpiStore)
    hipLaunchKernelGGL((dora_gemm_f32<AKC, BKC, kEpiStore>), grid, dim3(256), 0, st, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Fill KArgs from the problem; returns the total number of 64-deep K tiles.
int fill_args(const GemmProblem& p, KArgs& a) {
  a = KArgs{};
  a.M = (int)p.M;
  a.N = (int)p.N;
  int ns = 0, kt = 0;
  for (int s = 0; s < p.nseg; ++s) {
    if (p.seg[s].K <= 0) continue;
    a.a[ns] = reinterpret_cast<const uint16_t*>(p.seg[s].a);
    a.b[ns] = reinterpret_cast<const uint16_t*>(p.seg[s].b);
    a.lda[ns] = p.seg[s].lda;
    a.ldb[ns] = p.seg[s].ldb;
    a.K[ns] = (int)p.seg[s].K;
    kt += (int)cdiv64(p.seg[s].K, kBK);
    a.kt_end[ns] = kt;
    ++ns;
  }
  if (ns == 0) {  // empty K: C = 0 (one zero-length segment keeps the kernel uniform)
    a.K[0] = 0;
    a.kt_end[0] = 0;
    ns = 1;
  }
  for (int s = ns; s < 3; ++s) a.kt_end[s] = kt;
  a.nseg = ns;
  a.kt_total = kt;
  a.c = p.c;
  a.ldc = p.ldc;
  a.split_stride = p.split_stride;
  a.alpha = p.alpha;
  a.mag = p.mag;
  a.norm = p.norm;
  a.add = p.add;
  a.ld_add = p.ld_add;
  a.rowsq = p.rowsq;
  a.rowdot = p.rowdot;
  a.norm_out = p.norm_out;
  a.done = p.done;
  return kt;
}

hipError_t run(int cfg, int split, const GemmProblem& p, KArgs& a, int kt, hipStream_t st,
               bool out_f32) {
  const Cfg c = kCfgs[cfg];
  a.tiles_m = (int)cdiv64(p.M, c.bm);
  a.tiles_n = (int)cdiv64(p.N, c.bn);
  a.kt_per_split = split > 1 ? (kt + split - 1) / split : (kt > 0 ? kt : 1);
  if (a.kt_per_split < 1) a.kt_per_split = 1;
  a.nsplit = split;
  const dim3 grid(a.tiles_m * a.tiles_n * split);
  return launch_cfg(cfg, p.a_kcontig, p.b_kcontig, a, p.epi, out_f32, grid, st);
}

}  // namespace

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, int dtype, bool akc, bool bkc) {
  if (M <= 0 || N <= 0) return {-1, 1};
  const int64_t ktiles = cdiv64(K, kBK);
  if (dtype == kF32) {
    // 64 x 64 fp32-MFMA tiles (one wave per SIMD, latency-bound per workgroup; three
    // fit a CU): split K, down to one 64-deep step per split, up to ~768 workgroups
    const int64_t t = cdiv64(M, 64) * cdiv64(N, 64);
    int64_t split = std::min<int64_t>((768 + t - 1) / t, std::max<int64_t>(1, ktiles));
    return {-1, (int)std::max<int64_t>(1, std::min<int64_t>(split, 16))};
  }
  auto tiles = [&](int cfg) { return cdiv64(M, kCfgs[cfg].bm) * cdiv64(N, kCfgs[cfg].bn); };
  // Large outputs: 256 x 256 tiles (8 waves), then 256 x 128 (8 waves).  Two
  // transposed operands take the large tile only when they are copied straight
  // to LDS (two register-staged ones would not fit beside its accumulators).
  const bool both_mc = !akc && !bkc;
  if ((DORA_MC_DIRECT || !both_mc) && tiles(0) >= 256) return {0, 1};
  if (tiles(5) >= 256) return {5, 1};   // only when it still fills every CU
  // Skinny or small: 128 x 128 tiles, split along K into as many parts as one
  // round of workgroups holds (throughput grows with the workgroups resident
  // at once).  Two-stage tiles take two workgroups per CU (512 slots), the
  // three-stage ones one (256 slots); the plan whose round is fuller wins, and
  // a tie goes to fewer splits (less partial-sum traffic; one split needs no
  // reduction).  Measured on the d = 8192, r = 384 layer: x A^T and g_z B take
  // two stages and 5 splits, dB and dA three stages and no split.
  struct Cand {
    int cfg;
    int64_t slots;
  };
  const Cand cands[2] = {{2, 512}, {9, 256}};
  GemmPlan best = {2, 1};
  int64_t best_wgs = 0, best_cap = 1;   // fill = best_wgs / best_cap
  for (const Cand& c : cands) {
    const int64_t t = tiles(c.cfg);
    int64_t split = std::max<int64_t>(1, c.slots / t);
    split = std::min<int64_t>(split, std::max<int64_t>(1, ktiles / 8));
    split = std::min<int64_t>(split, 16);
    const int64_t wgs = t * split, cap = cdiv64(wgs, c.slots) * c.slots;
    if (best_wgs == 0 || wgs * best_cap > best_wgs * cap ||
        (wgs * best_cap == best_wgs * cap && split < best.split)) {
      best = {c.cfg, (int)split};
      best_wgs = wgs;
      best_cap = cap;
    }
  }
  return best;
}

GemmPlan plan_norm_projection(int64_t M, int64_t N, int64_t K, int64_t ld_max) {
  if (M <= 0 || N <= 0) return {-1, 1};
  // A rank of 257..384 fits one 128 x 384 tile: opA (W0) then crosses L2 once
  // per K split, and four splits of a d_out = 8192 layer make one workgroup
  // per CU (measured 62-65 us against 78-81 us for 128 x 128 tiles there).
  // Only while 384 rows of the widest operand span < 2^31 bytes.  Other ranks
  // keep the generic plan (128 x 128 tiles, measured fastest at r = 256).
  if (N > 256 && N <= 384 && ld_max * 2 * 384 < (int64_t(1) << 31)) {
    const int64_t tiles = cdiv64(M, kCfgs[6].bm);
    int64_t split = (256 + tiles / 2) / tiles;
    split = std::min<int64_t>(split, std::max<int64_t>(1, cdiv64(K, kBK) / 8));
    split = std::max<int64_t>(1, std::min<int64_t>(split, 16));
    return {6, (int)split};
  }
  // A rank of at most 64 would leave half of a 128-wide tile's columns empty:
  // 64 x 64 tiles (four waves, two stages), K split into about 384 workgroups
  // (one 64-deep step per split at least 8).  Measured at d_out = 2048,
  // d_in = 6144, r = 64: 11.7 us on 32 x 12 workgroups against 13.6-14.0 us for
  // the generic plan's 128 x 128 tiles (16 x 12).
  if (N <= 64) {
    const int64_t tiles = cdiv64(M, kCfgs[4].bm);
    int64_t split = std::max<int64_t>(1, (384 + tiles - 1) / tiles);
    split = std::min<int64_t>(split, std::max<int64_t>(1, cdiv64(K, kBK) / 8));
    split = std::max<int64_t>(1, std::min<int64_t>(split, 16));
    return {4, (int)split};
  }
  return plan_gemm(M, N, K, kBF16);
}

int64_t gemm_tile_rows(int cfg, int64_t M) {
  if (cfg < 0 || cfg >= kNumCfgs) return 0;
  return cdiv64(M, kCfgs[cfg].bm);
}

int64_t gemm_col_slots(int cfg, int64_t N) {
  if (cfg < 0 || cfg >= kNumCfgs) return 0;
  return cdiv64(N, kCfgs[cfg].bn);
}

size_t gemm_scratch_bytes(int64_t M, int64_t N, int64_t K, int dtype, bool akc, bool bkc) {
  const GemmPlan pl = plan_gemm(M, N, K, dtype, akc, bkc);
  return pl.split > 1 ? (size_t)pl.split * M * N * 4 : 0;
}

hipError_t gemm(const GemmProblem& p, int dtype, hipStream_t st, const char* label) {
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  KArgs a;
  const int kt = fill_args(p, a);
  int64_t K = 0;
  for (int s = 0; s < p.nseg; ++s) K += p.seg[s].K > 0 ? p.seg[s].K : 0;

  if (p.epi == kEpiNorm &&
      (dtype != kBF16 || !p.out_f32 || !p.a_kcontig || !p.b_kcontig || !p.rowsq || !p.rowdot ||
       !p.add || p.N % 4 != 0 || p.nseg < 1 || p.seg[0].K <= 0 || (p.norm_out && !p.done)))
    return hipErrorInvalidValue;
  if (dtype == kF32) {
    a.tiles_m = (int)cdiv64(p.M, 64);
    a.tiles_n = (int)cdiv64(p.N, 64);
    auto launch = [&](KArgs& args, int split, int epi) {
      args.kt_per_split = split > 1 ? (kt + split - 1) / split : (kt > 0 ? kt : 1);
      const dim3 grid(args.tiles_m * args.tiles_n, split);
      if (p.a_kcontig && p.b_kcontig) return launch_f32<true, true>(args, epi, grid, st);
      if (p.a_kcontig) return launch_f32<true, false>(args, epi, grid, st);
      if (p.b_kcontig) return launch_f32<false, true>(args, epi, grid, st);
      return launch_f32<false, false>(args, epi, grid, st);
    };
    if (p.split > 1 || p.out_f32) {   // caller-managed partial sums
      LaunchTimer timer(label, st);
      return launch(a, p.split < 1 ? 1 : p.split, p.epi);
    }
    const int split = p.force_split > 0 ? p.force_split : plan_gemm(p.M, p.N, K, dtype).split;
    const size_t need = (size_t)split * p.M * p.N * 4;
    if (split > 1 && (p.epi == kEpiStore || p.epi == kEpiCompose) && p.scratch &&
        p.scratch_bytes >= need && p.ldc == p.N) {
      KArgs b = a;   // float32 partials into scratch, then the fixed-order reduction
      b.c = p.scratch;
      b.ldc = p.N;
      b.split_stride = p.M * p.N;
      b.alpha = 1.f;
      {
        LaunchTimer timer(label, st);
        const hipError_t e = launch(b, split, kEpiStore);   // plain partials; the epilogue follows
        if (e != hipSuccess) return e;
      }
      LaunchTimer timer("splitk_reduce", st);
      const int64_t n4 = p.M * p.N / 4;
      const bool compose = p.epi == kEpiCompose;
      hipLaunchKernelGGL(dora_splitk_reduce, dim3((unsigned)cdiv64(n4, 256)), dim3(256), 0, st,
                         reinterpret_cast<const float*>(p.scratch), split, n4, p.M * p.N, p.alpha,
                         p.c, 0, compose ? p.mag : nullptr, 0, compose ? p.norm : nullptr,
                         (int)p.N);
      return hipGetLastError();
    }
    LaunchTimer timer(label, st);
    return launch(a, 1, p.epi);
  }

  int cfg = p.cfg;
  if (cfg < 0 || cfg >= kNumCfgs) cfg = plan_gemm(p.M, p.N, K, dtype, p.a_kcontig, p.b_kcontig).cfg;
  if (p.split > 1 || p.out_f32) {   // caller-managed partial sums (or a plain float32 output)
    LaunchTimer timer(label, st);
    return run(cfg, p.split < 1 ? 1 : p.split, p, a, kt, st, p.out_f32);
  }
  GemmPlan pl = plan_gemm(p.M, p.N, K, dtype, p.a_kcontig, p.b_kcontig);
  if (p.cfg >= 0) pl.cfg = cfg;
  if (p.force_split > 0) pl.split = p.force_split;
  const size_t need = (size_t)pl.split * p.M * p.N * 4;
  if (pl.split > 1 && (p.epi == kEpiStore || p.epi == kEpiCompose) && p.scratch &&
      p.scratch_bytes >= need && p.ldc == p.N) {
    // Split-K: float32 partials into scratch, then a fixed-order reduction
    // (which applies the compose epilogue when there is one).
    GemmProblem q = p;
    q.epi = kEpiStore;
    KArgs b = a;
    b.c = p.scratch;
    b.ldc = p.N;
    b.split_stride = p.M * p.N;
    b.alpha = 1.f;
    {
      LaunchTimer timer(label, st);
      const hipError_t e = run(pl.cfg, pl.split, q, b, kt, st, true);
      if (e != hipSuccess) return e;
    }
    const bool compose = p.epi == kEpiCompose;
    LaunchTimer timer("splitk_reduce", st);
    const int64_t n4 = p.M * p.N / 4;
    hipLaunchKernelGGL(dora_splitk_reduce, dim3((unsigned)cdiv64(n4, 256)), dim3(256), 0, st,
                       reinterpret_cast<const float*>(p.scratch), pl.split, n4, p.M * p.N, p.alpha,
                       p.c, 1, compose ? p.mag : nullptr, 1, compose ? p.norm : nullptr,
                       (int)p.N);
    return hipGetLastError();
  }
  // A 256 x 256 plan whose last round of workgroups is at most half full leaves
  // half the chip idle for that round.  When that round is whole tile columns,
  // those columns run as a second launch on 256 x 128 tiles (twice the
  // workgroups, each half as long); the epilogues act per output column or per
  // row, so a column slice of the problem computes exactly the same values.
  // Only for long K, where half a tile's time outweighs the extra launch
  // (27648-wide forward, K = 5376: 1995 -> 1983 us for the two launches).
  if (cfg == 0 && p.cfg < 0 && p.force_split <= 0 && K >= 2048 &&
      (p.epi == kEpiStore || p.epi == kEpiCompose || p.epi == kEpiMerge)) {
    const int64_t tm = cdiv64(p.M, 256), tn = cdiv64(p.N, 256), rem = (tm * tn) % 256;
    if (tm * tn > 256 && rem > 0 && rem <= 128 && rem % tm == 0) {
      const int64_t n_main = (tn - rem / tm) * 256;
      GemmProblem main_p = p, tail = p;
      main_p.N = n_main;
      main_p.cfg = 0;
      main_p.force_split = 1;
      tail.N = p.N - n_main;
      tail.cfg = 5;
      tail.force_split = 1;
      for (int sgi = 0; sgi < p.nseg; ++sgi) {
        const uint16_t* b = reinterpret_cast<const uint16_t*>(p.seg[sgi].b);
        if (b) tail.seg[sgi].b = p.b_kcontig ? b + n_main * p.seg[sgi].ldb : b + n_main;
      }
      tail.c = reinterpret_cast<uint16_t*>(p.c) + n_main;
      if (p.epi == kEpiCompose) {
        tail.mag = reinterpret_cast<const uint16_t*>(p.mag) + n_main;
        tail.norm = p.norm + n_main;
      }
      if (p.epi == kEpiMerge) tail.add = reinterpret_cast<const uint16_t*>(p.add) + n_main;
      const hipError_t e = gemm(main_p, dtype, st, label);
      if (e != hipSuccess) return e;
      return gemm(tail, dtype, st, label);
    }
  }
  LaunchTimer timer(label, st);
  return run(cfg, 1, p, a, kt, st, false);
}

}  // namespace dora
