// Dense contractions of the DoRA hot path on gfx950.
//
// bf16 operands run on the CDNA4 matrix cores (v_mfma_f32_32x32x16_bf16,
// float32 accumulation); float32 layers use a VALU tile kernel.  One kernel
// template covers every contraction of the path:
//   C[m, n] = alpha * sum over segments s, k < K_s of opA_s(m, k) * opB_s(n, k)
// where each operand is either K-contiguous or M/N-contiguous in memory, and
// up to three K segments are concatenated (e.g. [x | xs] . [W0 | B]^T).
//
// Tiling.  A workgroup owns a BM x BN output tile and walks K in 64-deep
// steps through a double-buffered LDS stage.  LDS rows are 64 bf16 = 128 B,
// split in eight 16-byte chunks whose order is XOR-swizzled by the row index
// ((row & 7) ^ ((row >> 3) & 7)) so that the eight rows a 16-byte-per-lane
// read or write touches land in distinct bank groups.  K-contiguous operands
// are copied global -> registers -> LDS with 16-byte loads; M/N-contiguous
// operands are loaded as 4(k) x 8(m) bf16 blocks and transposed in registers
// before the store, so the MFMA fragment reads are the same for both.
// Each wave computes a (BM/WM) x (BN/WN) sub-tile of 32x32 MFMA blocks.  The
// MFMA runs as D = opB-tile x opA-tile^T so that every lane ends up holding
// four consecutive output columns (8-byte bf16 / 16-byte f32 stores).
//
// Workgroups are dispatched round-robin over the 8 XCDs; the tile index is
// remapped so that consecutive tiles (which share operand panels) run on
// one XCD and share its L2, and tiles are walked in groups of 4 tile-rows.
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
  int kq_end[3];         // the same in 32-deep steps (ring kernel)
  int kq_total;
  int kq_per_split;
  int tiles_m, tiles_n;
  void* c;
  int64_t ldc;
  int64_t split_stride;
  float alpha;
  const void* mag;
  const float* norm;
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

// Operand views of one K segment (wave-uniform).
struct OpView {
  const uint16_t* p;
  int64_t ld;
  int K;
};

// ---- global -> LDS copies ---------------------------------------------------

// K-contiguous operand, R rows x 64 k, copied straight into LDS with
// buffer_load ... lds: one wave instruction fills 8 rows x 128 B, lane l
// takes row l/8 and physical chunk l%8, i.e. logical chunk (l%8) ^ swz(row).
// Per-lane byte offsets are fixed for a K segment and computed once
// (prepare); each 64-deep step only moves the scalar buffer base (issue).
template <int R, int NW>
struct DmaKC {
  static constexpr int kInstr = R / 8 / NW;   // per wave
  static_assert(R % (8 * NW) == 0, "rows must split evenly over the waves");
  const uint16_t* base;   // operand rows of this tile, k = 0
  int64_t ld;
  int64_t rows;           // valid rows in the tile
  int K;
  uint32_t off[kInstr];   // row * ld * 2 + chunk * 16
  uint32_t kcol[kInstr];  // chunk * 8 (k offset of the lane's 16 bytes)
  __device__ __forceinline__ void prepare(const OpView& v, int row0, int nrows, int wave,
                                          int lane) {
    rows = nrows - row0;
    if (rows > R) rows = R;
    base = v.p + (int64_t)row0 * v.ld;
    ld = v.ld;
    K = v.K;
#pragma unroll
    for (int i = 0; i < kInstr; ++i) {
      const int row = (wave * kInstr + i) * 8 + (lane >> 3);
      const int kc = (lane & 7) ^ swz(row);
      kcol[i] = (uint32_t)kc * 8u;
      // 32-bit arithmetic: a tile spans < 2^31 bytes (the library limits every dimension)
      off[i] = (uint32_t)row * (uint32_t)(v.ld * 2) + kcol[i] * 2u;
    }
  }
  __device__ __forceinline__ void issue(uint8_t* lds_tile, int k0, int wave) const {
    // rebased at column k0: rows past the tile's valid ones fall beyond the records
    const Rsrc rs = make_rsrc(base + k0, rows * ld * 2 - (int64_t)k0 * 2);
    const bool tail = k0 + kBK > K;   // uniform; only a segment's last step can be partial
#pragma unroll
    for (int i = 0; i < kInstr; ++i) {
      const int rbase = (wave * kInstr + i) * 8;
      const uint32_t o = (tail && (int)kcol[i] + k0 >= K) ? kOob : off[i];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(lds_tile + rbase * kRowBytes), 16, (int)o,
          0, 0, 0);
    }
  }
};

// M/N-contiguous operand: element (row, k) at p[k*ld + row].  Copied as
// blocks of 4 consecutive k x 8 consecutive rows (four 16-byte loads),
// transposed in registers into eight 8-byte row pieces.
template <int R, int NT>
struct RegMC {
  static constexpr int kRowChunks = R / 8;
  static constexpr int kBlocks = kRowChunks * (kBK / 4);
  static constexpr int kPer = (kBlocks + NT - 1) / NT;
  static_assert(kRowChunks % 8 == 0, "block order assumes a multiple of 64 rows");
  u32x4 v[kPer][4];
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
  const uint16_t* base;    // column row0 of the operand, k = 0
  int64_t ld;
  int K, row0, nrows;
  __device__ __forceinline__ void prepare(const OpView& o, int r0, int nr, int) {
    base = o.p + r0;
    ld = o.ld;
    K = o.K;
    row0 = r0;
    nrows = nr;
  }
  __device__ __forceinline__ void load(int k0, int tid) {
    int64_t krows = K - k0;
    if (krows > kBK) krows = kBK;
    // rebased at row k0; rows k >= K fall past the end of the records
    const Rsrc rs = make_rsrc(base + (int64_t)k0 * ld, krows * ld * 2 - (int64_t)row0 * 2);
    const uint32_t ld2 = (uint32_t)(ld * 2);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int b = tid + i * NT;
      int kq, rc;
      block_of(b, kq, rc);
      const bool ok = (kBlocks % NT == 0 || b < kBlocks) && row0 + rc * 8 < nrows;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        v[i][j] = bload16(rs, ok ? (uint32_t)(kq * 4 + j) * ld2 + (uint32_t)rc * 16u : kOob);
    }
  }
  __device__ __forceinline__ void store(uint8_t* lds, int tid) const {
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
        uint32_t lo, hi;
        if (mm & 1) {
          lo = (a0 >> 16) | (a1 & 0xffff0000u);
          hi = (a2 >> 16) | (a3 & 0xffff0000u);
        } else {
          lo = (a0 & 0xffffu) | (a1 << 16);
          hi = (a2 & 0xffffu) | (a3 << 16);
        }
        const int row = rc * 8 + mm;
        *reinterpret_cast<u32x2*>(lds + row * kRowBytes + ((chunk ^ swz(row)) << 4) + half * 8) =
            u32x2{lo, hi};
      }
    }
  }
};

// Per-operand copy policy: K-contiguous operands go global -> LDS directly,
// M/N-contiguous ones through registers (they are transposed on the way).
template <int R, int NT, bool KC>
struct Copier;
template <int R, int NT>
struct Copier<R, NT, true> {
  DmaKC<R, NT / 64> d;
  __device__ __forceinline__ void prepare(const OpView& o, int row0, int nrows, int tid, int wave,
                                          int lane) {
    d.prepare(o, row0, nrows, wave, lane);
  }
  __device__ __forceinline__ void issue(uint8_t* lds, int k0, int tid, int wave) {
    d.issue(lds, k0, wave);
  }
  __device__ __forceinline__ void commit(uint8_t*, int) {}
};
template <int R, int NT>
struct Copier<R, NT, false> {
  RegMC<R, NT> r;
  __device__ __forceinline__ void prepare(const OpView& o, int row0, int nrows, int tid, int,
                                          int) {
    r.prepare(o, row0, nrows, tid);
  }
  __device__ __forceinline__ void issue(uint8_t*, int k0, int tid, int) { r.load(k0, tid); }
  __device__ __forceinline__ void commit(uint8_t* lds, int tid) { r.store(lds, tid); }
};

__device__ __forceinline__ bf16x8 lds_frag(const uint8_t* lds, int row, int chunk) {
  return *reinterpret_cast<const bf16x8*>(lds + row * kRowBytes + ((chunk ^ swz(row)) << 4));
}

// Tile index -> (tile_m, tile_n), XCD-grouped, 8 tile-rows per group (an XCD's
// 32 CUs then hold an ~8 x 4 block of tiles and share its operand panels in L2).
// Returns tile_m in .x and tile_n in .y.
__device__ __forceinline__ int2 tile_coords(int tiles_m, int tiles_n) {
  int L = blockIdx.x;
  const int nwg = gridDim.x;
  if ((nwg & 7) == 0) L = (L & 7) * (nwg >> 3) + (L >> 3);
  constexpr int kGroup = 8;
  const int per_group = kGroup * tiles_n;
  const int g = L / per_group;
  const int first = g * kGroup;
  const int gsz = min(tiles_m - first, kGroup);
  const int rem = L - g * per_group;
  return make_int2(first + rem % gsz, rem / gsz);
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

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// s_waitcnt vmcnt(N) with the other counters left open (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Epilogue shared by the bf16 kernels: scale (and compose), then store.  bf16
// outputs are staged through LDS so that every store is a whole 16-byte piece
// of a row; float32 outputs (split-K partials) go straight out.
template <int BM, int BN, int WM, int WN, int EPI, bool OUT_F32>
__device__ __forceinline__ void gemm_epilogue(f32x16 (&acc)[BM / WM / 32][BN / WN / 32],
                                              uint8_t* smem, void* c, int64_t ldc,
                                              int64_t split_stride, float alpha, const void* mag,
                                              const float* nrm, int M, int N, int m0, int n0,
                                              int wave, int wm, int wn, int lane) {
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int MB = TM / 32, NB = TN / 32;
  constexpr int kStageLd = TN + 8;
  // Epilogue.  acc[i][j][v]: m = m0 + wm*TM + i*32 + lane%32,
  //                          n = n0 + wn*TN + j*32 + (v/4)*8 + (lane/32)*4 + v%4.
  void* cbase = OUT_F32 ? (void*)(reinterpret_cast<float*>(c) + blockIdx.y * split_stride)
                        : (void*)(reinterpret_cast<uint16_t*>(c) + blockIdx.y * split_stride);
  if constexpr (!OUT_F32) {
    // Stage the wave's tile in LDS (the K loop ended on a barrier, so every
    // stage is free), then write whole 16-byte pieces of contiguous rows.
    uint16_t* stg = reinterpret_cast<uint16_t*>(smem) + wave * TM * kStageLd;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int nl = j * 32 + g * 8 + (lane >> 5) * 4;
        const int n = n0 + wn * TN + nl;
        f32x4 gm1 = {0.f, 0.f, 0.f, 0.f};
        if (EPI == kEpiCompose && n < N) gm1 = gm1_4<true>(mag, nrm, n);
#pragma unroll
        for (int i = 0; i < MB; ++i) {
          const int ml = i * 32 + (lane & 31);
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float z = alpha * acc[i][j][g * 4 + e];
            v[e] = (EPI == kEpiCompose) ? z + gm1[e] * z : z;
          }
          *reinterpret_cast<u32x2*>(stg + ml * kStageLd + nl) =
              u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        }
      }
    }
    constexpr int kChunksPerRow = TN / 8;
#pragma unroll 4
    for (int c = lane; c < TM * kChunksPerRow; c += 64) {
      const int row = c / kChunksPerRow, ch = c - row * kChunksPerRow;
      const int m = m0 + wm * TM + row, n = n0 + wn * TN + ch * 8;
      const u32x4 val = *reinterpret_cast<const u32x4*>(stg + row * kStageLd + ch * 8);
      if (m < M && n < N)
        *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(cbase) + (int64_t)m * ldc + n) = val;
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

template <int BM, int BN, int WM, int WN, bool AKC, bool BKC, int EPI, bool OUT_F32, int NST = 2>
__global__ __launch_bounds__(WM * WN * 64) void dora_gemm_bf16(const KArgs p) {
  constexpr int NT = WM * WN * 64;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int MB = TM / 32, NB = TN / 32;
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(NST == 2 || (AKC && BKC), "deeper pipelines need both operands on the direct path");
  constexpr int ABYTES = BM * kRowBytes, BBYTES = BN * kRowBytes, STAGE = ABYTES + BBYTES;
  // bf16 outputs leave through LDS: each wave stages its TM x TN tile with rows
  // padded by 8 elements (conflict-free 8-byte writes, 16-byte aligned reads)
  constexpr int kStageLd = TN + 8;
  constexpr int kOutBytes = OUT_F32 ? 0 : WM * WN * TM * kStageLd * 2;
  constexpr int kSmem = NST * STAGE > kOutBytes ? NST * STAGE : kOutBytes;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kSmem];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % WM, wn = wave / WM;
  const int M = p.M, N = p.N;
  const int2 tc = tile_coords(p.tiles_m, p.tiles_n);
  const int m0 = tc.x * BM, n0 = tc.y * BN;
  const int kt_end0 = p.kt_end[0], kt_end1 = p.kt_end[1];
  const int kt_lo = blockIdx.y * p.kt_per_split;
  const int kt_hi = min(kt_lo + p.kt_per_split, p.kt_total);
  const uint16_t *a0 = p.a[0], *a1 = p.a[1], *a2 = p.a[2];
  const uint16_t *b0 = p.b[0], *b1 = p.b[1], *b2 = p.b[2];
  const int64_t lda0 = p.lda[0], lda1 = p.lda[1], lda2 = p.lda[2];
  const int64_t ldb0 = p.ldb[0], ldb1 = p.ldb[1], ldb2 = p.ldb[2];
  const int K0 = p.K[0], K1 = p.K[1], K2 = p.K[2];

  f32x16 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  Copier<BM, NT, AKC> ca;
  Copier<BN, NT, BKC> cb;
  int prep_seg = -1;   // K segment the copiers are prepared for
#define DORA_FETCH(KT, STAGE)                                                              \
  do {                                                                                     \
    const int s_ = (KT) < kt_end0 ? 0 : ((KT) < kt_end1 ? 1 : 2);                          \
    const int k0_ = ((KT) - (s_ == 0 ? 0 : (s_ == 1 ? kt_end0 : kt_end1))) * kBK;          \
    if (s_ != prep_seg) {                                                                  \
      prep_seg = s_;                                                                       \
      OpView va_, vb_;                                                                     \
      va_.p = s_ == 0 ? a0 : (s_ == 1 ? a1 : a2);                                          \
      va_.ld = s_ == 0 ? lda0 : (s_ == 1 ? lda1 : lda2);                                   \
      va_.K = s_ == 0 ? K0 : (s_ == 1 ? K1 : K2);                                          \
      vb_.p = s_ == 0 ? b0 : (s_ == 1 ? b1 : b2);                                          \
      vb_.ld = s_ == 0 ? ldb0 : (s_ == 1 ? ldb1 : ldb2);                                   \
      vb_.K = va_.K;                                                                       \
      ca.prepare(va_, m0, M, tid, wave, lane);                                             \
      cb.prepare(vb_, n0, N, tid, wave, lane);                                             \
    }                                                                                      \
    ca.issue((STAGE), k0_, tid, wave);                                                     \
    cb.issue((STAGE) + ABYTES, k0_, tid, wave);                                            \
  } while (0)

  // One LDS stage: 4 steps of 16 k.  Fragments for step kk+1 are read while
  // the MFMAs of step kk run (two register sets), so LDS latency hides behind
  // the matrix cores instead of stalling them.
  auto mma_stage = [&](const uint8_t* As) {
    const uint8_t* Bs = As + ABYTES;
    bf16x8 af[2][MB], bfg[2][NB];
    auto read = [&](int set, int kk) {
      const int ch = kk * 2 + (lane >> 5);
#pragma unroll
      for (int i = 0; i < MB; ++i) af[set][i] = lds_frag(As, wm * TM + i * 32 + (lane & 31), ch);
#pragma unroll
      for (int j = 0; j < NB; ++j) bfg[set][j] = lds_frag(Bs, wn * TN + j * 32 + (lane & 31), ch);
    };
    read(0, 0);
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int cs = kk & 1;
      if (kk + 1 < kBK / 16) read(cs ^ 1, kk + 1);
      // keep the reads of step kk+1 ahead of the MFMAs of step kk
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfg[cs][j], af[cs][i], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if constexpr (NST == 2) {
    if (kt_lo < kt_hi) {
      DORA_FETCH(kt_lo, smem);
      ca.commit(smem, tid);
      cb.commit(smem + ABYTES, tid);
      wait_vmem();
      __syncthreads();
      for (int kt = kt_lo; kt < kt_hi; ++kt) {
        const int cur = (kt - kt_lo) & 1;
        const bool more = kt + 1 < kt_hi;
        uint8_t* nx = smem + (cur ^ 1) * STAGE;
        if (more) DORA_FETCH(kt + 1, nx);
        mma_stage(smem + cur * STAGE);
        if (more) {
          ca.commit(nx, tid);
          cb.commit(nx + ABYTES, tid);
        }
        wait_vmem();
        __syncthreads();
      }
    }
  } else {
    // NST-stage ring, both operands copied straight to LDS: tile kt+NST-1 is
    // in flight while tile kt is multiplied.
    constexpr int kLoads = DmaKC<BM, NT / 64>::kInstr + DmaKC<BN, NT / 64>::kInstr;
    static_assert(kLoads * (NST - 2) < 64, "outstanding loads exceed vmcnt");
    if (kt_lo < kt_hi) {
#pragma unroll
      for (int i = 0; i < NST - 1; ++i)
        if (kt_lo + i < kt_hi) DORA_FETCH(kt_lo + i, smem + i * STAGE);
      wait_vmem();
      __syncthreads();
      int cur = 0;
      for (int kt = kt_lo; kt < kt_hi; ++kt) {
        const int ahead = kt + NST - 1;
        int slot = cur + NST - 1;
        if (slot >= NST) slot -= NST;
        if (ahead < kt_hi) DORA_FETCH(ahead, smem + slot * STAGE);
        mma_stage(smem + cur * STAGE);
        if (ahead < kt_hi)
          wait_vmem_le<kLoads * (NST - 2)>();   // tile kt+1 has landed
        else
          wait_vmem();
        __syncthreads();
        cur = cur + 1 == NST ? 0 : cur + 1;
      }
    }
  }
#undef DORA_FETCH

  gemm_epilogue<BM, BN, WM, WN, EPI, OUT_F32>(acc, smem, p.c, p.ldc, p.split_stride, p.alpha, p.mag,
                                                p.norm, M, N, m0, n0, wave, wm, wn, lane);
}

// ---- 32-deep ring pipeline (both operands K-contiguous) -----------------------
// Four LDS slots of 32-deep K steps.  Step q's copies go out two iterations
// before it is multiplied, in two halves placed between the MFMAs of the
// previous step, so the copy engine works while the matrix cores do; one
// barrier per step, without a memory fence, covers both the arrival of step
// q+1 and the reuse of the slot step q-1 occupied.
constexpr int kBKq = 32;            // K depth of one ring slot (bf16)
constexpr int kRowQ = kBKq * 2;     // 64-byte LDS rows: four 16-byte chunks
constexpr int kSlots = 4;

// Chunk permutation for 64-byte rows: eight (and sixteen) consecutive rows
// reading the same logical chunk land in distinct 16-byte bank slots of a
// 128-byte (and 256-byte) window.
__device__ __forceinline__ int swz4(int row) {
  return (((row >> 1) ^ (row >> 3)) & 1) | (((row >> 2) & 1) << 1);
}

__device__ __forceinline__ bf16x8 lds_frag4(const uint8_t* lds, int row, int chunk) {
  return *reinterpret_cast<const bf16x8*>(lds + row * kRowQ + ((chunk ^ swz4(row)) << 4));
}

// K-contiguous operand, R rows x 32 k per slot: one buffer_load ... lds fills
// 16 rows x 64 bytes; lane l takes row l/4 and physical chunk l%4.
template <int R, int NW>
struct DmaQ {
  static constexpr int kInstr = R / 16 / NW;   // per wave and slot
  static_assert(R % (16 * NW) == 0, "rows must split evenly over the waves");
  const uint16_t* base;
  int64_t ld;
  int64_t rows;
  int K;
  uint32_t off[kInstr];
  uint32_t kcol[kInstr];
  __device__ __forceinline__ void prepare(const uint16_t* p, int64_t ldv, int Kv, int row0,
                                          int nrows, int wave, int lane) {
    rows = nrows - row0;
    if (rows > R) rows = R;
    base = p + (int64_t)row0 * ldv;
    ld = ldv;
    K = Kv;
#pragma unroll
    for (int i = 0; i < kInstr; ++i) {
      const int row = (wave * kInstr + i) * 16 + (lane >> 2);
      const int kc = (lane & 3) ^ swz4(row);
      kcol[i] = (uint32_t)kc * 8u;
      off[i] = (uint32_t)row * (uint32_t)(ldv * 2) + kcol[i] * 2u;
    }
  }
  template <int I0, int I1>
  __device__ __forceinline__ void issue(uint8_t* lds_tile, int k0, int wave) const {
    if constexpr (I0 < I1) {
      const Rsrc rs = make_rsrc(base + k0, rows * ld * 2 - (int64_t)k0 * 2);
      const bool tail = k0 + kBKq > K;
#pragma unroll
      for (int i = I0; i < I1; ++i) {
        const int rbase = (wave * kInstr + i) * 16;
        const uint32_t o = (tail && (int)kcol[i] + k0 >= K) ? kOob : off[i];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (__attribute__((address_space(3))) void*)(lds_tile + rbase * kRowQ), 16, (int)o,
            0, 0, 0);
      }
    }
  }
};

// s_barrier with no memory fence: the waits it needs are explicit.  The asm
// memory clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void barrier_nofence() { asm volatile("s_barrier" ::: "memory"); }

template <int BM, int BN, int WM, int WN, int EPI, bool OUT_F32, bool SPLITQ = true>
__global__ __launch_bounds__(WM * WN * 64) void dora_gemm_ring(const KArgs p) {
  constexpr int NW = WM * WN;
  // SPLITQ: only the second half of the waves issue copies, so the first half
  // never stalls on the copy queue and keeps the matrix cores fed meanwhile.
  constexpr int NWC = SPLITQ ? NW / 2 : NW;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int MB = TM / 32, NB = TN / 32;
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be a multiple of 32");
  constexpr int ABYTES = BM * kRowQ, BBYTES = BN * kRowQ, STAGE = ABYTES + BBYTES;
  constexpr int kStageLd = TN + 8;
  constexpr int kOutBytes = OUT_F32 ? 0 : NW * TM * kStageLd * 2;
  constexpr int kSmem = kSlots * STAGE > kOutBytes ? kSlots * STAGE : kOutBytes;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kSmem];
  using DA = DmaQ<BM, NWC>;
  using DB = DmaQ<BN, NWC>;
  constexpr int kLoads = DA::kInstr + DB::kInstr;   // copies per wave and slot
  constexpr int kHalfA = (DA::kInstr + 1) / 2, kHalfB = (DB::kInstr + 1) / 2;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % WM, wn = wave / WM;
  const bool loader = !SPLITQ || wave >= NW - NWC;
  const int cwave = loader ? wave - (NW - NWC) : 0;   // index among the copying waves
  const int M = p.M, N = p.N;
  const int2 tc = tile_coords(p.tiles_m, p.tiles_n);
  const int m0 = __builtin_amdgcn_readfirstlane(tc.x * BM);
  const int n0 = __builtin_amdgcn_readfirstlane(tc.y * BN);
  const int kq_end0 = p.kq_end[0], kq_end1 = p.kq_end[1];
  const int kt_lo = blockIdx.y * p.kq_per_split;
  const int kt_hi = min(kt_lo + p.kq_per_split, p.kq_total);
  const uint16_t *a0 = p.a[0], *a1 = p.a[1], *a2 = p.a[2];
  const uint16_t *b0 = p.b[0], *b1 = p.b[1], *b2 = p.b[2];
  const int64_t lda0 = p.lda[0], lda1 = p.lda[1], lda2 = p.lda[2];
  const int64_t ldb0 = p.ldb[0], ldb1 = p.ldb[1], ldb2 = p.ldb[2];
  const int K0 = p.K[0], K1 = p.K[1], K2 = p.K[2];

  f32x16 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  DA ca;
  DB cb;
  int prep_seg = -1;
  int k0n = 0;   // k offset (within its segment) of the step being copied
  // Select the segment of step KT and prepare the copiers for it.
#define DORA_RING_SEG(KT)                                                                  \
  do {                                                                                     \
    const int s_ = (KT) < kq_end0 ? 0 : ((KT) < kq_end1 ? 1 : 2);                          \
    k0n = ((KT) - (s_ == 0 ? 0 : (s_ == 1 ? kq_end0 : kq_end1))) * kBKq;                   \
    if (s_ != prep_seg) {                                                                  \
      prep_seg = s_;                                                                       \
      const int Ks_ = s_ == 0 ? K0 : (s_ == 1 ? K1 : K2);                                  \
      ca.prepare(s_ == 0 ? a0 : (s_ == 1 ? a1 : a2), s_ == 0 ? lda0 : (s_ == 1 ? lda1 : lda2), \
                 Ks_, m0, M, cwave, lane);                                                 \
      cb.prepare(s_ == 0 ? b0 : (s_ == 1 ? b1 : b2), s_ == 0 ? ldb0 : (s_ == 1 ? ldb1 : ldb2), \
                 Ks_, n0, N, cwave, lane);                                                 \
    }                                                                                      \
  } while (0)
#define DORA_RING_COPY(SLOTP, H)                                                           \
  do {                                                                                     \
    if (loader) {                                                                          \
      if ((H) == 0) {                                                                      \
        ca.template issue<0, kHalfA>((SLOTP), k0n, cwave);                                 \
        cb.template issue<0, kHalfB>((SLOTP) + ABYTES, k0n, cwave);                        \
      } else {                                                                             \
        ca.template issue<kHalfA, DA::kInstr>((SLOTP), k0n, cwave);                        \
        cb.template issue<kHalfB, DB::kInstr>((SLOTP) + ABYTES, k0n, cwave);               \
      }                                                                                    \
    }                                                                                      \
  } while (0)

  bf16x8 af0[MB], bf0[NB], af1[MB], bf1[NB];
#define DORA_RING_READ(AF, BFR, SLOTP, KK)                                                 \
  do {                                                                                     \
    const int ch_ = (KK) * 2 + (lane >> 5);                                                \
    _Pragma("unroll") for (int i = 0; i < MB; ++i)                                         \
        AF[i] = lds_frag4((SLOTP), wm * TM + i * 32 + (lane & 31), ch_);                  \
    _Pragma("unroll") for (int j = 0; j < NB; ++j)                                         \
        BFR[j] = lds_frag4((SLOTP) + ABYTES, wn * TN + j * 32 + (lane & 31), ch_);        \
  } while (0)
#define DORA_RING_MMA(AF, BFR)                                                             \
  do {                                                                                     \
    _Pragma("unroll") for (int i = 0; i < MB; ++i)                                         \
        _Pragma("unroll") for (int j = 0; j < NB; ++j) acc[i][j] =                         \
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(BFR[j], AF[i], acc[i][j], 0, 0, 0);   \
  } while (0)

  if (kt_lo < kt_hi) {
    // Prologue: steps kt_lo .. kt_lo+2 into slots 0..2.
#pragma unroll
    for (int i = 0; i < kSlots - 1; ++i) {
      if (kt_lo + i < kt_hi) {
        DORA_RING_SEG(kt_lo + i);
        DORA_RING_COPY(smem + i * STAGE, 0);
        DORA_RING_COPY(smem + i * STAGE, 1);
      }
    }
    if (kt_lo + 2 < kt_hi) wait_vmem_le<2 * kLoads>();
    else if (kt_lo + 1 < kt_hi) wait_vmem_le<kLoads>();
    else wait_vmem_le<0>();
    barrier_nofence();
    DORA_RING_READ(af0, bf0, smem, 0);
    // One 32-deep step: MFMAs of its first half while its second half's fragments
    // arrive; then (if there is a next step) wait for that step, barrier, send the
    // first half of the copies of step kt+3 and read the next step's first
    // fragments; then the second half's MFMAs and the rest of the copies.
#define DORA_RING_STEP(HAS_NEXT, COPY, WAIT_LE)                                            \
  do {                                                                                     \
    const int rel_ = kt - kt_lo;                                                           \
    const uint8_t* cur_ = smem + (rel_ & 3) * STAGE;                                       \
    uint8_t* nxt_ = smem + ((rel_ + 1) & 3) * STAGE;                                       \
    uint8_t* cpy_ = smem + ((rel_ + 3) & 3) * STAGE;                                       \
    DORA_RING_READ(af1, bf1, cur_, 1);                                                     \
    __builtin_amdgcn_sched_barrier(0);                                                     \
    DORA_RING_MMA(af0, bf0);                                                               \
    __builtin_amdgcn_sched_barrier(0);                                                     \
    if (HAS_NEXT) {                                                                        \
      wait_vmem_le<(WAIT_LE)>();                                                           \
      barrier_nofence();                                                                   \
      if (COPY) {                                                                          \
        DORA_RING_SEG(kt + 3);                                                             \
        DORA_RING_COPY(cpy_, 0);                                                           \
      }                                                                                    \
      DORA_RING_READ(af0, bf0, nxt_, 0);                                                   \
    }                                                                                      \
    __builtin_amdgcn_sched_barrier(0);                                                     \
    DORA_RING_MMA(af1, bf1);                                                               \
    __builtin_amdgcn_sched_barrier(0);                                                     \
    if (COPY) DORA_RING_COPY(cpy_, 1);                                                     \
  } while (0)
    int kt = kt_lo;
    // steady state: a next step exists and step kt+3 is copied; step kt+2 may
    // still be in flight when step kt+1 is waited for
    for (; kt + 3 < kt_hi; ++kt) DORA_RING_STEP(true, true, kLoads);
    // the last (up to) three steps
    if (kt + 2 < kt_hi) {
      DORA_RING_STEP(true, false, kLoads);
      ++kt;
    }
    if (kt + 1 < kt_hi) {
      DORA_RING_STEP(true, false, 0);
      ++kt;
    }
    DORA_RING_STEP(false, false, 0);
#undef DORA_RING_STEP
    wait_vmem();
    __syncthreads();   // every wave is done with the ring before the epilogue reuses it
  }
#undef DORA_RING_SEG
#undef DORA_RING_COPY
#undef DORA_RING_READ
#undef DORA_RING_MMA

  gemm_epilogue<BM, BN, WM, WN, EPI, OUT_F32>(acc, smem, p.c, p.ldc, p.split_stride, p.alpha, p.mag,
                                                p.norm, M, N, m0, n0, wave, wm, wn, lane);
}

// ---- lean K-contiguous kernel ------------------------------------------------------
// Both operands K-contiguous, copied straight to LDS, two 64-deep stages.  The
// per-stage instruction stream is kept to the MFMAs, the fragment reads and the
// copies: buffer descriptors and per-lane offsets are set once per K segment and
// the K position travels in the scalar offset of each copy; only a segment's
// last, partial step checks K per lane; LDS read addresses are per-lane bases
// plus immediate offsets (the stage loop is unrolled by two).  With eight
// waves per CU every scalar or vector instruction in the loop competes with
// the MFMA issue, so this is what keeps the matrix cores busy.
template <int R, int NW>
struct LeanDma {
  static constexpr int kInstr = R / 8 / NW;   // 16-byte copies per lane and stage
  static_assert(R % (8 * NW) == 0, "rows must split evenly over the waves");
  Rsrc rs;                 // tile base at k = 0, records = valid rows * ld * 2
  uint32_t off[kInstr];    // row * ld * 2 + chunk * 16
  __device__ __forceinline__ void prepare(const uint16_t* p, int64_t ld, int row0, int nrows,
                                          int wave, int lane) {
    int64_t rows = nrows - row0;
    if (rows > R) rows = R;
    rs = make_rsrc(p + (int64_t)row0 * ld, rows * ld * 2);
#pragma unroll
    for (int i = 0; i < kInstr; ++i) {
      const int row = (wave * kInstr + i) * 8 + (lane >> 3);
      const int kc = (lane & 7) ^ swz(row);
      off[i] = (uint32_t)row * (uint32_t)(ld * 2) + (uint32_t)kc * 16u;
    }
  }
  // Full step at byte column kbytes of the segment.
  __device__ __forceinline__ void issue(uint8_t* lds_tile, int kbytes, int wave) const {
#pragma unroll
    for (int i = 0; i < kInstr; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(lds_tile + (wave * kInstr + i) * 8 * kRowBytes),
          16, (int)off[i], kbytes, 0, 0);
  }
  // Partial step: chunks at or beyond K read as zeros.
  __device__ __forceinline__ void issue_tail(uint8_t* lds_tile, int kbytes, int K, int wave,
                                             int lane) const {
#pragma unroll
    for (int i = 0; i < kInstr; ++i) {
      const int row = (wave * kInstr + i) * 8 + (lane >> 3);
      const int kc = (lane & 7) ^ swz(row);
      const bool in = kbytes / 2 + kc * 8 < K;
      // kOob + kbytes stays below 2^32 and beyond every record count
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(lds_tile + (wave * kInstr + i) * 8 * kRowBytes),
          16, (int)(in ? off[i] : kOob), kbytes, 0, 0);
    }
  }
};

template <int BM, int BN, int WM, int WN, int EPI, bool OUT_F32>
__global__ __launch_bounds__(WM * WN * 64) void dora_gemm_kc(const KArgs p) {
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int MB = TM / 32, NB = TN / 32;
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be a multiple of 32");
  // LDS: [A stage 0 | A stage 1 | B stage 0 | B stage 1], so that every fragment
  // read is a per-lane base plus an offset that fits the 16-bit immediate.
  constexpr int ABYTES = BM * kRowBytes, BBYTES = BN * kRowBytes, STAGE = ABYTES + BBYTES;
  constexpr int BBASE = 2 * ABYTES;
  static_assert(ABYTES + (BM > 64 ? 64 * kRowBytes : 0) < 65536 && BBYTES < 65536,
                "stage offsets must fit the LDS immediate");
  constexpr int kStageLd = TN + 8;
  constexpr int kOutBytes = OUT_F32 ? 0 : NW * TM * kStageLd * 2;
  constexpr int kSmem = 2 * STAGE > kOutBytes ? 2 * STAGE : kOutBytes;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kSmem];
  using DA = LeanDma<BM, NW>;
  using DB = LeanDma<BN, NW>;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % WM, wn = wave / WM;
  const int M = p.M, N = p.N;
  const int2 tc = tile_coords(p.tiles_m, p.tiles_n);
  const int m0 = __builtin_amdgcn_readfirstlane(tc.x * BM);
  const int n0 = __builtin_amdgcn_readfirstlane(tc.y * BN);
  const int kt_lo = blockIdx.y * p.kt_per_split;
  const int kt_hi = min(kt_lo + p.kt_per_split, p.kt_total);

  f32x16 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

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

  const int kt_end0 = p.kt_end[0], kt_end1 = p.kt_end[1], kt_end2 = p.kt_end[2];
  const uint16_t *a0 = p.a[0], *a1 = p.a[1], *a2 = p.a[2];
  const uint16_t *b0 = p.b[0], *b1 = p.b[1], *b2 = p.b[2];
  const int64_t lda0 = p.lda[0], lda1 = p.lda[1], lda2 = p.lda[2];
  const int64_t ldb0 = p.ldb[0], ldb1 = p.ldb[1], ldb2 = p.ldb[2];
  const int K0 = p.K[0], K1 = p.K[1], K2 = p.K[2];

  // Copies of K tile KT (relative tile KR of its segment) into stage buffer SB.
#define DORA_KC_FETCH(KR, SB)                                                              \
  do {                                                                                     \
    const int kb_ = (KR) * (kBK * 2);                                                      \
    uint8_t* sa_ = smem + (SB) * ABYTES;                                                   \
    uint8_t* sb_ = smem + BBASE + (SB) * BBYTES;                                           \
    if (partial && (KR) == last) {                                                         \
      ca.issue_tail(sa_, kb_, Ks, wave, lane);                                             \
      cb.issue_tail(sb_, kb_, Ks, wave, lane);                                             \
    } else {                                                                               \
      ca.issue(sa_, kb_, wave);                                                            \
      cb.issue(sb_, kb_, wave);                                                            \
    }                                                                                      \
  } while (0)

  bf16x8 af[2][MB], bfr[2][NB];
#define DORA_KC_READ(SET, SB, KK)                                                          \
  do {                                                                                     \
    _Pragma("unroll") for (int i = 0; i < MB; ++i) af[SET][i] =                            \
        *reinterpret_cast<const bf16x8*>(smem + ra[i & 1][KK] + (i >> 1) * 64 * kRowBytes + \
                                         (SB) * ABYTES);                                   \
    _Pragma("unroll") for (int j = 0; j < NB; ++j) bfr[SET][j] =                           \
        *reinterpret_cast<const bf16x8*>(smem + rb[j & 1][KK] + (j >> 1) * 64 * kRowBytes + \
                                         (SB) * BBYTES);                                   \
  } while (0)
  // One stage: four 16-deep steps, fragments of step kk+1 read during step kk.
#define DORA_KC_MMA(SB)                                                                    \
  do {                                                                                     \
    DORA_KC_READ(0, SB, 0);                                                                \
    _Pragma("unroll") for (int kk = 0; kk < 4; ++kk) {                                     \
      if (kk < 3) {                                                                        \
        if (kk & 1) DORA_KC_READ(0, SB, kk + 1);                                           \
        else DORA_KC_READ(1, SB, kk + 1);                                                  \
      }                                                                                    \
      __builtin_amdgcn_sched_barrier(0);                                                   \
      _Pragma("unroll") for (int i = 0; i < MB; ++i)                                       \
          _Pragma("unroll") for (int j = 0; j < NB; ++j) acc[i][j] =                       \
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[kk & 1][j], af[kk & 1][i],      \
                                                      acc[i][j], 0, 0, 0);                 \
      __builtin_amdgcn_sched_barrier(0);                                                   \
    }                                                                                      \
  } while (0)

  // Segments one after the other; the two-stage pipeline restarts at each
  // (at most two restarts per launch), so within a segment the copy state is
  // loop-invariant and stays in scalar registers.
#pragma unroll 1
  for (int seg = 0; seg < 3; ++seg) {
    const int s_lo = seg == 0 ? 0 : (seg == 1 ? kt_end0 : kt_end1);
    const int s_hi = seg == 0 ? kt_end0 : (seg == 1 ? kt_end1 : kt_end2);
    const int lo = max(kt_lo, s_lo), hi = min(kt_hi, s_hi);
    if (lo >= hi) continue;
    const int Ks = seg == 0 ? K0 : (seg == 1 ? K1 : K2);
    const bool partial = (Ks % kBK) != 0;
    const int last = s_hi - 1 - s_lo;   // relative index of the segment's last tile
    DA ca;
    DB cb;
    ca.prepare(seg == 0 ? a0 : (seg == 1 ? a1 : a2), seg == 0 ? lda0 : (seg == 1 ? lda1 : lda2),
               m0, M, wave, lane);
    cb.prepare(seg == 0 ? b0 : (seg == 1 ? b1 : b2), seg == 0 ? ldb0 : (seg == 1 ? ldb1 : ldb2),
               n0, N, wave, lane);
    const int r_lo = lo - s_lo, r_hi = hi - s_lo;
    DORA_KC_FETCH(r_lo, 0);
    wait_vmem();
    barrier_nofence();
    for (int kr = r_lo; kr < r_hi; kr += 2) {
      if (kr + 1 < r_hi) DORA_KC_FETCH(kr + 1, 1);
      DORA_KC_MMA(0);
      wait_vmem();
      barrier_nofence();
      if (kr + 1 >= r_hi) break;
      if (kr + 2 < r_hi) DORA_KC_FETCH(kr + 2, 0);
      DORA_KC_MMA(1);
      wait_vmem();
      barrier_nofence();
    }
  }
#undef DORA_KC_FETCH
#undef DORA_KC_READ
#undef DORA_KC_MMA

  gemm_epilogue<BM, BN, WM, WN, EPI, OUT_F32>(acc, smem, p.c, p.ldc, p.split_stride, p.alpha, p.mag,
                                                p.norm, M, N, m0, n0, wave, wm, wn, lane);
}

// float32 layers: 64x64 tiles, 16-deep K steps, 4x4 outputs per thread.
template <bool AKC, bool BKC, int EPI>
__global__ __launch_bounds__(256) void dora_gemm_f32(const KArgs p) {
  constexpr int BM = 64, BN = 64, BKF = 16;
  __shared__ float As[BKF][BM + 4];
  __shared__ float Bs[BKF][BN + 4];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int2 tc = tile_coords(p.tiles_m, p.tiles_n);
  const int m0 = tc.x * BM, n0 = tc.y * BN;
  float acc[4][4] = {};
  const int kt_total = p.kt_total;   // in 64-deep units, shared with the bf16 path
  const int kt_lo = blockIdx.y * p.kt_per_split;
  const int kt_hi = min(kt_lo + p.kt_per_split, kt_total);
  for (int kt = kt_lo; kt < kt_hi; ++kt) {
    const int s = kt < p.kt_end[0] ? 0 : (kt < p.kt_end[1] ? 1 : 2);
    const int kbase = (kt - (s == 0 ? 0 : (s == 1 ? p.kt_end[0] : p.kt_end[1]))) * kBK;
    const float* a = reinterpret_cast<const float*>(s == 0 ? p.a[0] : (s == 1 ? p.a[1] : p.a[2]));
    const float* b = reinterpret_cast<const float*>(s == 0 ? p.b[0] : (s == 1 ? p.b[1] : p.b[2]));
    const int64_t lda = s == 0 ? p.lda[0] : (s == 1 ? p.lda[1] : p.lda[2]);
    const int64_t ldb = s == 0 ? p.ldb[0] : (s == 1 ? p.ldb[1] : p.ldb[2]);
    const int Ks = s == 0 ? p.K[0] : (s == 1 ? p.K[1] : p.K[2]);
    for (int ks = 0; ks < kBK; ks += BKF) {
      const int k0 = kbase + ks;
      if (k0 >= Ks) break;
      for (int e = tid; e < BM * BKF; e += 256) {
        const int mm = AKC ? e / BKF : e % BM, kk = AKC ? e % BKF : e / BM;
        const int gm = m0 + mm, gk = k0 + kk;
        float va = 0.f;
        if (gm < p.M && gk < Ks)
          va = AKC ? a[(int64_t)gm * lda + gk] : a[(int64_t)gk * lda + gm];
        As[kk][mm] = va;
        const int nn = BKC ? e / BKF : e % BN, kb = BKC ? e % BKF : e / BN;
        const int gn = n0 + nn, gk2 = k0 + kb;
        float vb = 0.f;
        if (gn < p.N && gk2 < Ks)
          vb = BKC ? b[(int64_t)gn * ldb + gk2] : b[(int64_t)gk2 * ldb + gn];
        Bs[kb][nn] = vb;
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < BKF; ++kk) {
        float ra[4], rb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ra[i] = As[kk][ty * 4 + i];
#pragma unroll
        for (int j = 0; j < 4; ++j) rb[j] = Bs[kk][tx * 4 + j];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(ra[i], rb[j], acc[i][j]);
      }
      __syncthreads();
    }
  }
  float* c = reinterpret_cast<float*>(p.c) + blockIdx.y * p.split_stride;
  const int n = n0 + tx * 4;
  if (n >= p.N) return;
  f32x4 gm1 = {0.f, 0.f, 0.f, 0.f};
  if (EPI == kEpiCompose) gm1 = gm1_4<false>(p.mag, p.norm, n);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= p.M) continue;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float z = p.alpha * acc[i][e];
      v[e] = (EPI == kEpiCompose) ? z + gm1[e] * z : z;
    }
    store4<true>(c, p.ldc, m, n, v[0], v[1], v[2], v[3]);
  }
}

// ---- split-K reduction ----------------------------------------------------------
// out[i] = alpha * sum_{z < S} part[z][i] over M*N elements, fixed order.
__global__ __launch_bounds__(256) void dora_splitk_reduce(const float* part, int S, int64_t n4,
                                                          int64_t stride, float alpha, void* out,
                                                          int out_bf16) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  f32x4 acc = reinterpret_cast<const f32x4*>(part)[i];
  for (int z = 1; z < S; ++z) {
    const f32x4 v = reinterpret_cast<const f32x4*>(part + z * stride)[i];
    acc += v;
  }
  acc *= alpha;
  if (out_bf16)
    reinterpret_cast<u32x2*>(out)[i] = u32x2{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
  else
    reinterpret_cast<f32x4*>(out)[i] = acc;
}

// ---- host-side dispatch -----------------------------------------------------

// Tile configurations: BM x BN workgroup tile, WM x WN waves.
// `ring`: the 32-deep four-slot pipeline (both operands K-contiguous only).
struct Cfg {
  int bm, bn, wm, wn;
  bool ring;
};
constexpr Cfg kCfgs[] = {
    {256, 256, 2, 4, false},   // 0: 8 waves, 128x64 per wave
    {256, 128, 2, 2, false},   // 1: 4 waves, 128x64 per wave
    {128, 128, 2, 2, false},   // 2: 4 waves, 64x64 per wave
    {128, 256, 2, 2, false},   // 3: 4 waves, 64x128 per wave
    {64, 64, 2, 2, false},     // 4: 4 waves, 32x32 per wave
    {256, 128, 4, 2, false},   // 5: 8 waves, 64x64 per wave
    {256, 256, 2, 4, true},    // 6: ring, 8 waves, 128x64 per wave
    {128, 128, 2, 2, true},    // 7: ring, 4 waves, 64x64 per wave
    {256, 128, 4, 2, true},    // 8: ring, 8 waves, 64x64 per wave
    {128, 256, 2, 2, true},    // 9: ring, 4 waves, 64x128 per wave
    {256, 256, 2, 4, true},    // 10: ring, every wave copies
    {128, 128, 2, 2, true},    // 11: ring, every wave copies
    {256, 256, 2, 4, true},    // 12: lean K-contiguous, 8 waves, 128x64 per wave
    {128, 128, 2, 2, true},    // 13: lean K-contiguous, 4 waves, 64x64 per wave
    {256, 128, 4, 2, true},    // 14: lean K-contiguous, 8 waves, 64x64 per wave
};
constexpr int kNumCfgs = sizeof(kCfgs) / sizeof(kCfgs[0]);

template <int BM, int BN, int WM, int WN, bool AKC, bool BKC, int NST = 2>
hipError_t launch_bf16(const KArgs& a, int epi, bool out_f32, dim3 grid, hipStream_t st) {
  const dim3 block(WM * WN * 64);
  if (out_f32) {
    hipLaunchKernelGGL((dora_gemm_bf16<BM, BN, WM, WN, AKC, BKC, kEpiStore, true, NST>), grid,
                       block, 0, st, a);
    return hipGetLastError();
  }
  if constexpr (AKC && BKC) {   // the compose epilogue belongs to the forward (K-contiguous) GEMM
    if (epi == kEpiCompose) {
      hipLaunchKernelGGL((dora_gemm_bf16<BM, BN, WM, WN, AKC, BKC, kEpiCompose, false, NST>), grid,
                         block, 0, st, a);
      return hipGetLastError();
    }
  } else {
    if (epi != kEpiStore) return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL((dora_gemm_bf16<BM, BN, WM, WN, AKC, BKC, kEpiStore, false, NST>), grid,
                     block, 0, st, a);
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_layout(bool akc, bool bkc, const KArgs& a, int epi, bool out_f32, dim3 grid,
                         hipStream_t st) {
  if (akc && bkc) return launch_bf16<BM, BN, WM, WN, true, true>(a, epi, out_f32, grid, st);
  if (akc && !bkc) return launch_bf16<BM, BN, WM, WN, true, false>(a, epi, out_f32, grid, st);
  if (!akc && !bkc) return launch_bf16<BM, BN, WM, WN, false, false>(a, epi, out_f32, grid, st);
  return hipErrorInvalidValue;
}

template <int BM, int BN, int WM, int WN, bool SQ = true>
hipError_t launch_ring(bool akc, bool bkc, const KArgs& a, int epi, bool out_f32, dim3 grid,
                       hipStream_t st) {
  if (!(akc && bkc)) return hipErrorInvalidValue;
  const dim3 block(WM * WN * 64);
  if (out_f32)
    hipLaunchKernelGGL((dora_gemm_ring<BM, BN, WM, WN, kEpiStore, true, SQ>), grid, block, 0, st, a);
  else if (epi == kEpiCompose)
    hipLaunchKernelGGL((dora_gemm_ring<BM, BN, WM, WN, kEpiCompose, false, SQ>), grid, block, 0, st,
                       a);
  else
    hipLaunchKernelGGL((dora_gemm_ring<BM, BN, WM, WN, kEpiStore, false, SQ>), grid, block, 0, st, a);
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_kc(bool akc, bool bkc, const KArgs& a, int epi, bool out_f32, dim3 grid,
                     hipStream_t st) {
  if (!(akc && bkc)) return hipErrorInvalidValue;
  const dim3 block(WM * WN * 64);
  if (out_f32)
    hipLaunchKernelGGL((dora_gemm_kc<BM, BN, WM, WN, kEpiStore, true>), grid, block, 0, st, a);
  else if (epi == kEpiCompose)
    hipLaunchKernelGGL((dora_gemm_kc<BM, BN, WM, WN, kEpiCompose, false>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((dora_gemm_kc<BM, BN, WM, WN, kEpiStore, false>), grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_cfg(int cfg, bool akc, bool bkc, const KArgs& a, int epi, bool out_f32, dim3 grid,
                      hipStream_t st) {
  switch (cfg) {
    case 0: return launch_layout<256, 256, 2, 4>(akc, bkc, a, epi, out_f32, grid, st);
    case 1: return launch_layout<256, 128, 2, 2>(akc, bkc, a, epi, out_f32, grid, st);
    case 2: return launch_layout<128, 128, 2, 2>(akc, bkc, a, epi, out_f32, grid, st);
    case 3: return launch_layout<128, 256, 2, 2>(akc, bkc, a, epi, out_f32, grid, st);
    case 4: return launch_layout<64, 64, 2, 2>(akc, bkc, a, epi, out_f32, grid, st);
    case 5: return launch_layout<256, 128, 4, 2>(akc, bkc, a, epi, out_f32, grid, st);
    case 6: return launch_ring<256, 256, 2, 4>(akc, bkc, a, epi, out_f32, grid, st);
    case 7: return launch_ring<128, 128, 2, 2>(akc, bkc, a, epi, out_f32, grid, st);
    case 8: return launch_ring<256, 128, 4, 2>(akc, bkc, a, epi, out_f32, grid, st);
    case 9: return launch_ring<128, 256, 2, 2>(akc, bkc, a, epi, out_f32, grid, st);
    case 10: return launch_ring<256, 256, 2, 4, false>(akc, bkc, a, epi, out_f32, grid, st);
    case 11: return launch_ring<128, 128, 2, 2, false>(akc, bkc, a, epi, out_f32, grid, st);
    case 12: return launch_kc<256, 256, 2, 4>(akc, bkc, a, epi, out_f32, grid, st);
    case 13: return launch_kc<128, 128, 2, 2>(akc, bkc, a, epi, out_f32, grid, st);
    case 14: return launch_kc<256, 128, 4, 2>(akc, bkc, a, epi, out_f32, grid, st);

    default: return hipErrorInvalidValue;
  }
}

template <bool AKC, bool BKC>
hipError_t launch_f32(const KArgs& a, int epi, dim3 grid, hipStream_t st) {
  if (epi == kEpiCompose)
    hipLaunchKernelGGL((dora_gemm_f32<AKC, BKC, kEpiCompose>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((dora_gemm_f32<AKC, BKC, kEpiStore>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Fill KArgs from the problem; returns the total number of 64-deep K tiles.
int fill_args(const GemmProblem& p, KArgs& a) {
  a = KArgs{};
  a.M = (int)p.M;
  a.N = (int)p.N;
  int ns = 0, kt = 0, kq = 0;
  for (int s = 0; s < p.nseg; ++s) {
    if (p.seg[s].K <= 0) continue;
    a.a[ns] = reinterpret_cast<const uint16_t*>(p.seg[s].a);
    a.b[ns] = reinterpret_cast<const uint16_t*>(p.seg[s].b);
    a.lda[ns] = p.seg[s].lda;
    a.ldb[ns] = p.seg[s].ldb;
    a.K[ns] = (int)p.seg[s].K;
    kt += (int)cdiv64(p.seg[s].K, kBK);
    kq += (int)cdiv64(p.seg[s].K, kBKq);
    a.kt_end[ns] = kt;
    a.kq_end[ns] = kq;
    ++ns;
  }
  if (ns == 0) {  // empty K: C = 0 (one zero-length segment keeps the kernel uniform)
    a.K[0] = 0;
    a.kt_end[0] = 0;
    a.kq_end[0] = 0;
    ns = 1;
  }
  for (int s = ns; s < 3; ++s) {
    a.kt_end[s] = kt;
    a.kq_end[s] = kq;
  }
  a.nseg = ns;
  a.kt_total = kt;
  a.kq_total = kq;
  a.c = p.c;
  a.ldc = p.ldc;
  a.split_stride = p.split_stride;
  a.alpha = p.alpha;
  a.mag = p.mag;
  a.norm = p.norm;
  return kt;
}

hipError_t run(int cfg, int split, const GemmProblem& p, KArgs& a, int kt, hipStream_t st,
               bool out_f32) {
  const Cfg c = kCfgs[cfg];
  a.tiles_m = (int)cdiv64(p.M, c.bm);
  a.tiles_n = (int)cdiv64(p.N, c.bn);
  a.kt_per_split = split > 1 ? (kt + split - 1) / split : (kt > 0 ? kt : 1);
  if (a.kt_per_split < 1) a.kt_per_split = 1;
  const int kq = a.kq_total;
  a.kq_per_split = split > 1 ? (kq + split - 1) / split : (kq > 0 ? kq : 1);
  if (a.kq_per_split < 1) a.kq_per_split = 1;
  const dim3 grid(a.tiles_m * a.tiles_n, split);
  return launch_cfg(cfg, p.a_kcontig, p.b_kcontig, a, p.epi, out_f32, grid, st);
}

}  // namespace

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, int dtype, bool akc, bool bkc) {
  if (dtype == kF32 || M <= 0 || N <= 0) return {-1, 1};
  const int64_t ktiles = cdiv64(K, kBK);
  auto tiles = [&](int cfg) { return cdiv64(M, kCfgs[cfg].bm) * cdiv64(N, kCfgs[cfg].bn); };
  const bool direct = akc && bkc;
  // Large outputs: 256 x 256 tiles (8 waves), then 256 x 128 (8 waves); pairs of
  // K-contiguous operands run the ring pipeline.
  if (tiles(0) >= 256) return {direct ? 12 : 0, 1};
  if (tiles(5) >= 200) return {direct ? 14 : 5, 1};
  // Skinny or small, split along K.  Measured on the d = 8192, r = 384 layer:
  // K-contiguous pairs do best on 128 x 128 tiles at ~384 workgroups, pairs
  // with a transposed operand on 256 x 256 tiles at ~256 workgroups.
  const int cfg = direct ? 13 : 0;
  const int64_t target = direct ? 384 : 256;
  const int64_t t = tiles(cfg);
  int64_t split = (target + t / 2) / t;
  split = std::min<int64_t>(split, std::max<int64_t>(1, ktiles / 8));
  split = std::max<int64_t>(1, std::min<int64_t>(split, 16));
  return {cfg, (int)split};
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

  if (dtype == kF32) {
    LaunchTimer timer(label, st);
    a.tiles_m = (int)cdiv64(p.M, 64);
    a.tiles_n = (int)cdiv64(p.N, 64);
    const int split = p.split < 1 ? 1 : p.split;
    a.kt_per_split = split > 1 ? (kt + split - 1) / split : (kt > 0 ? kt : 1);
    const dim3 grid(a.tiles_m * a.tiles_n, split);
    if (p.a_kcontig && p.b_kcontig) return launch_f32<true, true>(a, p.epi, grid, st);
    if (p.a_kcontig) return launch_f32<true, false>(a, p.epi, grid, st);
    if (p.b_kcontig) return launch_f32<false, true>(a, p.epi, grid, st);
    return launch_f32<false, false>(a, p.epi, grid, st);
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
  if (pl.split > 1 && p.epi == kEpiStore && p.scratch && p.scratch_bytes >= need) {
    // Split-K: float32 partials into scratch, then a fixed-order reduction.
    KArgs b = a;
    b.c = p.scratch;
    b.ldc = p.N;
    b.split_stride = p.M * p.N;
    b.alpha = 1.f;
    {
      LaunchTimer timer(label, st);
      const hipError_t e = run(pl.cfg, pl.split, p, b, kt, st, true);
      if (e != hipSuccess) return e;
    }
    if (p.ldc != p.N) return hipErrorInvalidValue;
    LaunchTimer timer("splitk_reduce", st);
    const int64_t n4 = p.M * p.N / 4;
    hipLaunchKernelGGL(dora_splitk_reduce, dim3((unsigned)cdiv64(n4, 256)), dim3(256), 0, st,
                       reinterpret_cast<const float*>(p.scratch), pl.split, n4, p.M * p.N, p.alpha,
                       p.c, 1);
    return hipGetLastError();
  }
  LaunchTimer timer(label, st);
  return run(cfg, 1, p, a, kt, st, false);
}

}  // namespace dora
