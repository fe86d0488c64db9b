// Grouped SwiGLU experts over the ragged per-expert row blocks of the
// permuted matrix X.
//
// Method: page "MoE 与专家并行", section "从稠密 FFN 到 MoE", eq.
// FFN(u) = W_down (SiLU(W_gate u) * W_up u) with W_gate, W_up in R^{f x h} and
// W_down in R^{h x f}; section "专家计算：padding、block-sparse 与 grouped GEMM":
// one launch runs every expert's GEMM, scheduled by tiles from the per-expert
// row counts and offsets, with gate and up merged into one GEMM, the SiLU
// product in its epilogue, and a second GEMM for down.
//
// Kernels (gfx950): C[M, N] = A[M, K] W[N, K]^T with both operands
// K-contiguous and float32 accumulation, on v_mfma_f32_32x32x16_bf16 for bf16
// operands, or on v_mfma_f32_32x32x64_f8f6f4 for the FP8 (E4M3) up-projection
// of section "低精度通信" (DeepSeek-V3: activations quantised to FP8 with
// power-of-two scales before dispatch, FP8 up-projection, BF16 combine).  A
// workgroup of NW waves (NW/2 along M x 2 along N) owns a BM x 256 output
// tile; each wave a (2 BM / NW) x 128 block of 32 x 32 MFMA tiles.
//
// Operand pipeline.  K advances in steps of 128 bytes per row (64 bf16 or
// 128 FP8 elements), so every LDS-direct copy instruction (16 bytes per lane)
// moves eight whole 128-byte lines; on this part such copies sustain about
// twice the per-CU rate of 64-byte row pieces.  LDS holds a ring of N_A A
// slots and N_B B slots (2 + 3 at BM = 256, 3 + 3 at BM = 128).  Step j reads
// A_j and B_j; before its last K slice every wave waits for its copies of
// A_{j+1} and B_{j+1}, meets the others at one barrier, and then reuses the
// slots of step j for A_{j+N_A} and B_{j+N_B}.  Inside a step, each wave runs
// the MFMAs of one K slice while reading the fragments of the next from LDS.
// The slots are separate LDS arrays and the loop is unrolled over the ring's
// period, so the compiler can tell the copies in flight from the slots being
// read.  The forward bf16 products (gemm_chain_kernel) keep the ring running
// from one tile to the next: the copies past a tile's last step fetch the
// next tile's first steps; the FP8 and backward products refill it per tile.
//
// LDS rows are 128 bytes (8 chunks of 16).  gfx950 serves a 16-byte LDS read
// for 16 lanes per clock from 64 four-byte banks; storing logical chunk c of
// row r at chunk c ^ ((r >> 1) & 7) makes the 16 rows of one fragment read
// cover all banks once.  A bf16 fragment is one chunk per lane, an FP8
// fragment two.
//
// Gate/up tile: LDS B rows 0..127 are W_gate rows n0..n0+127 and rows
// 128..255 the W_up rows with the same indices, so each lane holds the gate
// and the up value of one output element and the epilogue writes
// a = SiLU(g) * u (rounded to bf16) directly; with FP8 operands g and u are
// first multiplied by the row scale of A and the row scales of W_gate / W_up.
// Ragged rows: an m-tile never crosses an expert boundary and only stores its
// valid rows.  Its A buffer resource ends at its last valid row, so copies of
// the rows past it read zero without memory traffic, and each wave skips the
// MFMAs of its 32-row blocks without valid rows.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "blocks.hpp"
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

// Waves per GEMM workgroup: 4 along M x 2 along N.  Two waves share each SIMD,
// so one can issue MFMAs while the other waits for LDS or a barrier.
constexpr int kWaves = 8;

constexpr int BN = 256, BK = 64, GN = 8;
// Operand element types: every K step moves 128 bytes of each row, i.e. 64
// bf16 or 128 FP8 elements, in 4 or 2 MFMA K slices.
typedef int v8i __attribute__((ext_vector_type(8)));
template <bool F8>
struct Elt {
  static constexpr int kBytes = F8 ? 1 : 2;    // bytes per element
  static constexpr int kStep = 128 / kBytes;   // K elements per step
  static constexpr int kSlices = F8 ? 2 : 4;   // MFMA K slices per step
  using Frag = std::conditional_t<F8, v8i, bf16x8>;
};

struct GemmParams {
  const void* A;         // [rows][K], experts' row blocks back to back (bf16 or FP8)
  const int32_t* offset; // [E+1]
  const int32_t* tmap;   // tile map: [E+1] first m-tile of each expert, then the
                         // per-m-tile table (see tile_map_kernel)
  const void* W0;        // gate/up: W_gate [E][N][K]; down: W_down [E][N][K]
  const void* W1;        // gate/up: W_up
  bf16* C;               // [rows][Nout]
  const float* sa;       // FP8: [rows] power-of-two scale of each A row
  const float* sw0;      // FP8: [E][N] scale of each W0 row
  const float* sw1;      // FP8: [E][N] scale of each W1 row
  int E, K, N, Nout;     // N: rows of each weight matrix (f or h)
  int ntiles, mtmax;
  float* part;           // K-split partial tiles: [grid][BM * BN] float32
  int split_max;         // most K chunks a tail tile is split into
  int grid;              // workgroups of the GEMM launch (a multiple of 8)
  bf16* C2 = nullptr;    // gate/up: also store the pre-activations g and u,
                         // [rows][2 Nout] (g in columns 0..Nout-1, u after)
  // weight gradients (gemm_wgrad_kernel): M columns of A per expert (K is
  // then A's row pitch and Nout B's)
  int M = 0;
  // BT kernels (weights stored [K][N]): W0 holds K rows 0..K0-1 of each
  // expert's [K][N] operand and W1 the rest ([E][K0][N] and [E][K-K0][N])
  int K0 = 0;
  int gn = GN;  // n-tiles per group of the tile numbering
};

// A K chunk of a tail tile (see xcd_share); ks == 1: a whole tile.
struct KSplit {
  int kbeg, ksteps;  // 128-byte K steps of this chunk
  int ks;            // chunks of the tile
  float* slot;       // where this chunk's float32 partial goes (ks > 1)
};

// Work of one XCD (workgroup i runs on XCD i % 8): a contiguous slice of the
// tile numbering, done in rounds of nloc tiles.  When the slice is only a few
// rounds long, the rem < nloc tiles left for the last round are each cut into
// ks K chunks so that round keeps about nloc workgroups busy; with many
// rounds the idle part of the last one matters little and the reduction
// would cost more than it saves.
constexpr int kSplitRounds = 4;  // split the tail only after at most this many full rounds
struct XcdShare {
  int tbeg, full, rem, ks, nloc;
};
__device__ __forceinline__ XcdShare xcd_share(int total, int xcd, int grid, int KT,
                                              int split_max) {
  XcdShare x;
  x.nloc = grid >> 3;
  const int per = (total + 7) >> 3;
  x.tbeg = xcd * per;
  const int ntile = max(0, min(total, x.tbeg + per) - x.tbeg);
  x.full = ntile / x.nloc * x.nloc;
  x.rem = ntile - x.full;
  x.ks = (x.rem > 0 && x.full <= kSplitRounds * x.nloc)
             ? max(1, min(min(split_max, x.nloc / x.rem), KT))
             : 1;
  return x;
}

// Tile t of the numbering: groups of p.gn n-tiles (GN unless the host widens
// them), m-tile major inside a group.
// The m-tile's expert, first row and valid rows come from one 8-byte entry of
// the tile map's table.
struct TileAt {
  int e, nt, row0, nvalid;
};
__device__ __forceinline__ const int2* mtile_table(const int32_t* tmap, int E) {
  return reinterpret_cast<const int2*>(tmap + ((E + 2) & ~1));
}
template <int BM>
__device__ __forceinline__ TileAt tile_at(const GemmParams& p, int t, int mtiles) {
  const int g = t / (mtiles * p.gn);
  const int r = t - g * mtiles * p.gn;
  const int gw = min(p.gn, p.ntiles - g * p.gn);
  const int mt = r / gw;
  const int2 m = mtile_table(p.tmap, p.E)[mt];
  TileAt x;
  x.nt = g * p.gn + r % gw;
  x.e = m.y & 0xffff;
  x.row0 = m.x;
  x.nvalid = m.y >> 16;
  return x;
}

// Float32 partial of a K chunk, in the accumulators' own per-thread order:
// float4 group q of thread i at slot + 4 * (q * blockDim + i).
template <int RBLK, int NW>
__device__ __forceinline__ float4* part_at(float* slot, int q) {
  return reinterpret_cast<float4*>(slot) + (size_t)q * 64 * NW + threadIdx.x;
}

// Epilogue: the wave's (2 BM / NW) x 128 block.  The MFMAs take the weight
// fragment as their first operand, so each 32x32 accumulator is the block's
// transpose: lane holds output row (lane % 32) and output columns
// 8 * g + 4 * (lane / 32) + t in acc[4 * g + t], g, t = 0..3.  Each run of 4
// columns goes out as one 8-byte store.  Gate/up: a = SiLU(g) * u from the
// gate and up halves, which sit in the same lane and register.
template <int BM, int NW, bool GATEUP, bool F8>
__device__ __forceinline__ void store_tile(const GemmParams& p, const floatx16 (&acc)[(2 * BM / NW) / 32][4],
                                           const TileAt& ta) {
  constexpr int WR = 2 * BM / NW, RBLK = WR / 32;
  const int nt = ta.nt, row0 = ta.row0, nvalid = ta.nvalid;
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));  // keeps the row addressing below out of the main loop
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1, l32 = lane & 31, khalf = lane >> 5;
#pragma unroll
  for (int i = 0; i < RBLK; ++i) {
    const int r = wm * WR + i * 32 + l32;
    if (r >= nvalid) continue;
    bf16* crow = p.C + (size_t)(row0 + r) * p.Nout;
    const float sa = F8 ? p.sa[row0 + r] : 1.f;
#pragma unroll
    for (int j = 0; j < (GATEUP ? 2 : 4); ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // Nout is a multiple of 4: a run is all inside or all past the end
        const int col = (GATEUP ? nt * 128 + wn * 64 : nt * BN + wn * 128) + j * 32 + 8 * g + 4 * khalf;
        if (col >= p.Nout) continue;
        float y[4], sg[4] = {1.f, 1.f, 1.f, 1.f}, su[4] = {1.f, 1.f, 1.f, 1.f};
        if (F8) {  // power-of-two scales: the products below are exact
          const float4 a = *reinterpret_cast<const float4*>(p.sw0 + (size_t)ta.e * p.N + col);
          sg[0] = sa * a.x; sg[1] = sa * a.y; sg[2] = sa * a.z; sg[3] = sa * a.w;
          if (GATEUP) {
            const float4 b = *reinterpret_cast<const float4*>(p.sw1 + (size_t)ta.e * p.N + col);
            su[0] = sa * b.x; su[1] = sa * b.y; su[2] = sa * b.z; su[3] = sa * b.w;
          }
        }
        float gp[4], up[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          if (GATEUP) {
            // SiLU(g) u = g u / (1 + e^-g), with the hardware reciprocal
            // (1 ulp) instead of a correctly rounded division: the product is
            // rounded to bf16 next
            const float gv = acc[i][j][4 * g + t] * sg[t], uv = acc[i][j + 2][4 * g + t] * su[t];
            y[t] = gv * uv * __builtin_amdgcn_rcpf(1.f + __expf(-gv));
            gp[t] = gv;
            up[t] = uv;
          } else {
            y[t] = acc[i][j][4 * g + t] * sg[t];  // sg = 1 for bf16 operands
          }
        }
        *reinterpret_cast<uint2*>(crow + col) = make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
        if (GATEUP && p.C2) {
          bf16* prow = p.C2 + (size_t)(row0 + r) * 2 * p.Nout;
          *reinterpret_cast<uint2*>(prow + col) =
              make_uint2(pack_bf16x2(gp[0], gp[1]), pack_bf16x2(gp[2], gp[3]));
          *reinterpret_cast<uint2*>(prow + p.Nout + col) =
              make_uint2(pack_bf16x2(up[0], up[1]), pack_bf16x2(up[2], up[3]));
        }
      }
    }
  }
}


template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}


// LDS slots of the copy pipeline: NA slots of A tiles and NB of B tiles
// (2 or 3 each); operand X of step j is copied N_X steps ahead.
struct Ring {
  bf16* a[3];
  bf16* b[3];
};

// Epilogue through LDS (weight gradients, whose tiles have few K steps and
// whose 256 x 256 outputs are the bulk of the kernel's traffic).  After the K
// loop the ring is idle: its slots A0, A1, B0, B1 hold the tile's rows 0-63,
// 64-127, 128-191, 192-255 as bf16, 512 bytes a row, 16-byte chunk c of row r
// at c ^ (r mod 32) (the 32 rows a wave writes at once then fall into
// different banks).  Each wave then stores 32 whole rows, two per
// instruction, 16 bytes per lane, so every store covers full cache lines.
template <int BM, int NW>
__device__ __forceinline__ void store_tile_staged(const GemmParams& p,
                                                  const floatx16 (&acc)[(2 * BM / NW) / 32][4],
                                                  const TileAt& ta, const Ring& L) {
  static_assert(BM == 256 && NW == 8, "staged epilogue: 256 x 256 tiles, 8 waves");
  constexpr int RBLK = 2;
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1, l32 = lane & 31, kh = lane >> 5;
  char* const slot[4] = {reinterpret_cast<char*>(L.a[0]), reinterpret_cast<char*>(L.a[1]),
                         reinterpret_cast<char*>(L.b[0]), reinterpret_cast<char*>(L.b[1])};
  char* const mine = slot[wm];  // rows wm * 64 .. + 63
#pragma unroll
  for (int i = 0; i < RBLK; ++i) {
    const int r = i * 32 + l32;  // row within the slot; r mod 32 = l32
    char* rowp = mine + r * 512;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = wn * 16 + j * 4 + g;  // logical chunk: columns 8c .. 8c + 7
        *reinterpret_cast<uint2*>(rowp + ((c ^ l32) * 16) + 8 * kh) =
            make_uint2(pack_bf16x2(acc[i][j][4 * g], acc[i][j][4 * g + 1]),
                       pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]));
      }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  barrier_only();
  // wave w stores rows 32 w .. 32 w + 31 (in slot w / 2)
  const char* src = slot[wm];
  const int col = ta.nt * BN + l32 * 8;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int rr = (wave & 1) * 32 + 2 * q + kh;  // row within the slot
    const int r = wm * 64 + rr;                   // row within the tile
    const uint4 v = *reinterpret_cast<const uint4*>(src + rr * 512 + ((l32 ^ (rr & 31)) * 16));
    // non-temporal: the gradient is not read again here, and a stream of
    // whole lines that bypasses L2's retention leaves the operand panels
    // there (5% on the Mixtral shape; the streaming kernel's stores, which
    // cover a line only across instructions, ran 3.6x slower so marked)
    if (r < ta.nvalid && col < p.Nout)
      __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w},
                                  reinterpret_cast<u32x4*>(p.C + (size_t)(ta.row0 + r) * p.Nout + col));
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  barrier_only();  // the slots are free for the next unit's copies
}

// Copy sources of one unit of work (a tile, or one K chunk of a tail tile):
// buffer resources over its valid A rows and its weight panels, and its range
// of K steps.  A's resource ends at the last valid row, so copies of
// rows past it read zero without touching memory (their outputs are never
// stored).
struct TileSrc {
  __amdgpu_buffer_rsrc_t rA, rB0, rB1;
  int kbeg, KT;
  int kt0;   // BT: K steps taken from W0 (the later ones come from W1)
  int klast; // copies of steps past the end reload step klast (in bounds,
             // never read), so that every step issues the same copies
};
template <bool GATEUP, bool F8, bool BT = false>
__device__ __forceinline__ TileSrc tile_src(const GemmParams& p, const TileAt& ta,
                                            const KSplit& ksp) {
  TileSrc s;
  if constexpr (BT) {  // weights [K][N]: the panel is columns n0.. of K rows
    const size_t pitch = (size_t)p.N * 2, nb = (size_t)ta.nt * BN * 2;
    const char* A = static_cast<const char*>(p.A);
    s.rA = make_rsrc(A + (size_t)ta.row0 * p.K * 2, (size_t)ta.nvalid * p.K * 2);
    const char* W0 = static_cast<const char*>(p.W0);
    const char* W1 = static_cast<const char*>(p.W1);
    const size_t b0 = (size_t)p.K0 * pitch, b1 = (size_t)(p.K - p.K0) * pitch;
    s.rB0 = make_rsrc(W0 + (size_t)ta.e * b0 + nb, b0 - nb);
    s.rB1 = p.K > p.K0 ? make_rsrc(W1 + (size_t)ta.e * b1 + nb, b1 - nb) : s.rB0;
    s.kbeg = ksp.kbeg;
    s.KT = ksp.ksteps;
    s.kt0 = p.K0 / BK;
    s.klast = s.KT - 1;
    return s;
  }
  const size_t rb = (size_t)p.K * Elt<F8>::kBytes;  // bytes per row
  const char* A = static_cast<const char*>(p.A);
  s.rA = make_rsrc(A + (size_t)ta.row0 * rb, (size_t)ta.nvalid * rb);
  const size_t n0 = (size_t)ta.nt * (GATEUP ? 128 : BN);
  const char* W0 = static_cast<const char*>(p.W0);
  const char* W1 = static_cast<const char*>(p.W1);
  s.rB0 = make_rsrc(W0 + ((size_t)ta.e * p.N + n0) * rb, (size_t)(p.N - n0) * rb);
  s.rB1 = GATEUP ? make_rsrc(W1 + ((size_t)ta.e * p.N + n0) * rb, (size_t)(p.N - n0) * rb)
                 : s.rB0;
  s.kbeg = ksp.kbeg;
  s.KT = ksp.ksteps;
  s.klast = s.KT - 1;
  return s;
}

// This wave's share of the copies of one K step.  Lane i of 8-row group g
// fills LDS row 8g + i/8, physical chunk i%8, with logical chunk
// (i%8) ^ ((row >> 1) & 7).  The per-lane offsets depend on K only.
//
// BT: the weight operand is stored [K][N] (N contiguous).  Its K step is then
// 64 rows of the tile's 256 columns, 512 bytes each, kept in that layout:
// copy instruction q of a wave fills k-rows 2 (wave + NW q) and the next,
// lane i physical chunk i % 32 of row 2 (wave + NW q) + i / 32 with logical
// chunk (i % 32) ^ trswz(row); fragments are read with the transposing LDS
// load (see gemm_tile).
__device__ __forceinline__ constexpr int trswz(int kr) { return (kr & 3) << 2; }

//
// AT: the same for the A operand, stored [K][M] (weight gradients), its K
// step 64 rows of the tile's BM columns.
template <int BM, int NW, bool GATEUP, bool F8, bool BT = false, bool AT = false>
struct CopyPlan {
  static constexpr int AG = BM / (8 * NW);  // 8-row A groups copied per wave per step
  static constexpr int BG = BN / (8 * NW);  // 8-row B groups copied per wave per step
  int wave;
  int voA[AG], voB[BG];
  int astep, bstep;  // AT / BT: bytes of one K step (64 rows) of A / of the weight panel
  // K: row length of the K-contiguous operands; N, M: row lengths (elements)
  // of a [K][N] weight operand (BT) and a [K][M] A operand (AT)
  __device__ __forceinline__ explicit CopyPlan(int K, int N = 0, int M = 0) {
    // the wave index is uniform: keep it (and all copy addressing) in SGPRs
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, lrow = lane >> 3;
#pragma unroll
    for (int j = 0; j < AG; ++j) {
      if constexpr (AT) {  // BM / 8 chunks per k-row
        constexpr int CPR = BM / 8, RPI = 64 / CPR;  // chunks per row, rows per copy
        const int kr = RPI * (wave + NW * j) + lane / CPR;
        voA[j] = kr * M * 2 + (((lane % CPR) ^ trswz(kr)) * 16);
      } else {
        const int r = 8 * (wave + NW * j) + lrow;
        voA[j] = r * K * Elt<F8>::kBytes + (((lane & 7) ^ ((r >> 1) & 7)) * 16);
      }
    }
    astep = BK * M * 2;
#pragma unroll
    for (int j = 0; j < BG; ++j) {
      if constexpr (BT) {
        const int kr = 2 * (wave + NW * j) + (lane >> 5);
        voB[j] = kr * N * 2 + (((lane & 31) ^ trswz(kr)) * 16);
      } else {
        // gate/up: groups 0..15 are W_gate rows, 16..31 (j >= BG/2) the W_up rows
        const int g = wave + NW * j;
        const int r = 8 * g + lrow;                       // LDS row
        const int pr = GATEUP ? 8 * (g & 15) + lrow : r;  // row in the weight panel
        voB[j] = pr * K * Elt<F8>::kBytes + (((lane & 7) ^ ((r >> 1) & 7)) * 16);
      }
    }
    bstep = BK * N * 2;
  }
  // step j past the end reloads the last step (in bounds, never read), so
  // every step issues the same number of copies
  __device__ __forceinline__ void issueA(const TileSrc& s, bf16* as, int j) const {
    const int kb = (s.kbeg + min(j, s.klast)) * (AT ? astep : 128);
#pragma unroll
    for (int q = 0; q < AG; ++q) dma16(s.rA, as + (wave + NW * q) * 8 * BK, voA[q], kb);
  }
  __device__ __forceinline__ void issueB(const TileSrc& s, bf16* bs, int j) const {
    if constexpr (BT) {
      const int st = s.kbeg + min(j, s.klast);
      const bool second = st >= s.kt0;
      const int kb = (second ? st - s.kt0 : st) * bstep;
#pragma unroll
      for (int q = 0; q < BG; ++q)
        dma16(second ? s.rB1 : s.rB0, bs + (wave + NW * q) * 8 * BK, voB[q], kb);
      return;
    }
    const int kb = (s.kbeg + min(j, s.klast)) * 128;
#pragma unroll
    for (int q = 0; q < BG; ++q)
      dma16((GATEUP && q >= BG / 2) ? s.rB1 : s.rB0, bs + (wave + NW * q) * 8 * BK, voB[q], kb);
  }
  // the first N_A A steps and N_B B steps of a unit, into slot phase 0
  template <int NA, int NB>
  __device__ __forceinline__ void prologue(const TileSrc& s, const Ring& L) const {
    issueA(s, L.a[0], 0);
    issueB(s, L.b[0], 0);
    issueA(s, L.a[1], 1);
    issueB(s, L.b[1], 1);
    if (NA == 3) issueA(s, L.a[2], 2);
    if (NB == 3) issueB(s, L.b[2], 2);
  }
};

// R: the 32-row blocks of this wave that hold valid rows (the first R of its
// RBLK); a wave with R < RBLK skips the fragment reads and MFMAs of the others
// (their accumulators stay zero and their rows are never stored) but issues
// the same copies and meets the same barriers as the rest of the workgroup.
template <int BM, int NW, bool GATEUP, bool F8, int R, int NA, int NB, bool BT, bool AT,
          bool STAGED, class Next>
__device__ __forceinline__ void gemm_tile(const GemmParams& p,
                                          const CopyPlan<BM, NW, GATEUP, F8, BT, AT>& cp,
                                          const TileSrc& src, const Ring& L, const TileAt& ta,
                                          const KSplit& ksp, Next&& next) {
  constexpr int WM = NW / 2;         // waves along M (2 along N)
  constexpr int WR = BM / WM;        // rows per wave
  constexpr int RBLK = WR / 32;      // 32-row MFMA blocks per wave
  constexpr int AG = CopyPlan<BM, NW, GATEUP, F8, BT, AT>::AG;
  constexpr int BG = CopyPlan<BM, NW, GATEUP, F8, BT, AT>::BG;
  constexpr int NSL = Elt<F8>::kSlices;  // MFMA K slices per step
  constexpr int FC = F8 ? 2 : 1;         // 16-byte chunks per fragment and lane
  using Frag = typename Elt<F8>::Frag;
  static_assert(AG >= 1 && BG >= 2 && RBLK >= 1, "tile shape");
  const int wave = cp.wave;
  const int lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int KT = src.KT;
  auto issueA = [&](bf16* as, int j) { cp.issueA(src, as, j); };
  auto issueB = [&](bf16* bs, int j) { cp.issueB(src, bs, j); };

  // ---- fragments: lane reads row (lane % 32) of each 32-row block, logical
  // chunks FC * (2 * slice + lane / 32) + 0..FC-1 of the step's 8.  The A and
  // B fragments of a slice cover the same K elements in the same lane and
  // byte positions, which is all the MFMA's dot products need.
  const int l32 = lane & 31, khalf = lane >> 5;
  const int sw = (l32 >> 1) & 7;  // (row >> 1) & 7 of every fragment row of this lane
  int aoff[RBLK], boff[4];  // byte offsets of this lane's rows in a slot
  // transposing read (see below): lane 4 q + m of each 16-lane group
  // addresses k-row q of the slice's 8 (+ 4 for the second half) and columns
  // 4 (m % 4) .. +3 of its 16; width: the tile's columns
  auto tr_off = [&](int width, int x0) {
    const int l16 = lane & 15, kr = 8 * khalf + (l16 >> 2);
    const int c = (x0 + 16 * ((lane >> 4) & 1) + 4 * (l16 & 3)) >> 3;
    return kr * (width * 2) + ((c ^ trswz(kr)) * 16) + 8 * (l16 & 1);
  };
#pragma unroll
  for (int i = 0; i < RBLK; ++i)
    aoff[i] = AT ? tr_off(BM, wm * WR + i * 32) : (wm * WR + i * 32 + l32) * 128;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (BT) {
      boff[j] = tr_off(BN, wn * 128 + j * 32);
    } else {
      const int r = GATEUP ? ((j < 2 ? 0 : 128) + wn * 64 + (j & 1) * 32 + l32)
                           : (wn * 128 + j * 32 + l32);
      boff[j] = r * 128;
    }
  }
  static_assert(R >= 0 && R <= RBLK, "active blocks");

  floatx16 acc[RBLK][4];
#pragma unroll
  for (int i = 0; i < RBLK; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  Frag fa[2][RBLK], fb[2][4];
  // one fragment: FC chunks of 16 bytes of a row, at physical chunks c ^ sw
  auto frag = [&](const bf16* slot, int off, int c0) {
    const char* row = reinterpret_cast<const char*>(slot) + off;
    if constexpr (F8) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(row + ((c0 ^ sw) * 16));
      const u32x4 y = *reinterpret_cast<const u32x4*>(row + (((c0 + 1) ^ sw) * 16));
      return Frag{(int)x[0], (int)x[1], (int)x[2], (int)x[3],
                  (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
    } else {
      return *reinterpret_cast<const Frag*>(row + ((c0 ^ sw) * 16));
    }
  };
  // Fragment of an operand stored [K][columns] (AT, BT): two transposing
  // 8-byte reads (ds_read_b64_tr_b16) of k-rows 16 slice + 8 khalf + (0..3,
  // 4..7).  Within each 16-lane group, lane i gets element i % 4 of the 8
  // bytes that lanes 4 q + i / 4 (q = 0..3) address; with the addresses of
  // tr_off, lane i receives column i of the group's 16 at 4 consecutive k,
  // so the lane holds column l32 at k = 16 slice + 8 khalf + 0..7, as a
  // K-contiguous fragment does.
  auto fragT = [&](const bf16* slot, int off, int slice, int width) {
    typedef short v4s __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4s lds_v4s;
    const char* q = reinterpret_cast<const char*>(slot) + off + slice * (16 * width * 2);
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(q));
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(q + 4 * width * 2));
    const v4s v[2] = {lo, hi};
    bf16x8 r;
    __builtin_memcpy(&r, v, 16);
    return r;
  };
  auto fetch = [&](const bf16* as, const bf16* bs, int slice, int st) {
    const int c0 = FC * (2 * slice + khalf);
#pragma unroll
    for (int i = 0; i < R; ++i) {
      if constexpr (AT) fa[st][i] = fragT(as, aoff[i], slice, BM);
      else fa[st][i] = frag(as, aoff[i], c0);
    }
#pragma unroll
    for (int j = 0; j < (R > 0 ? 4 : 0); ++j) {
      if constexpr (BT) fb[st][j] = fragT(bs, boff[j], slice, BN);
      else fb[st][j] = frag(bs, boff[j], c0);
    }
  };
  auto mfmas = [&](int st) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (F8)  // format codes 0, 0: both operands E4M3; no block scales
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              fb[st][j], fa[st][i], acc[i][j], 0, 0, 0, 0, 0, 0);
        else
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[st][j], fa[st][i], acc[i][j],
                                                              0, 0, 0);
      }
    }
  };
  // order for the scheduler: MFMAs interleaved with the next fragment reads
  // and, after the barrier, with the copies (groups: 0x008 MFMA, 0x100 LDS
  // read, 0x020 global read incl. LDS copies)
  constexpr int NM = R * 4, NR = R > 0 ? R * (AT ? 2 : FC) + 4 * (BT ? 2 : FC) : 0;
  constexpr int NC = AG + BG;
  constexpr int CPM = NM > 0 ? (NC + NM - 1) / NM : NC;  // copies placed after each MFMA
  constexpr int RPM = NM > 0 ? (NR + NM - 1) / NM : NR;  // LDS reads placed after each MFMA
  auto order = [&]() {
    if (R == 0) return;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (m * RPM < NR) __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);
    }
  };
  auto order_copies = [&]() {
    if (R == 0) return;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (m * CPM < NC) __builtin_amdgcn_sched_group_barrier(0x020, CPM, 0);
      if (m * RPM < NR) __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);
    }
  };
  // Step j on slots (as, bs); (nas, nbs) hold step j + 1.  On entry fa/fb[0]
  // hold slice 0 of step j.
  auto step = [&](int j, bf16* as, bf16* bs, const bf16* nas, const bf16* nbs) {
#pragma unroll
    for (int sl = 0; sl + 1 < NSL; ++sl) {
      fetch(as, bs, sl + 1, (sl + 1) & 1);
      mfmas(sl & 1);
      order();
    }
    // A_{j+1} and B_{j+1} have landed; copies of step j + 2 (issued last)
    // may still be in flight
    wait_vm<(NA == 3 ? AG : 0) + (NB == 3 ? BG : 0)>();
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave is done reading (as, bs)
    barrier_only();
    // into the slots just read: the operand copied 2 steps ahead first
    if (NA == 2) issueA(as, j + 2);
    issueB(bs, j + NB);
    if (NA == 3) issueA(as, j + 3);
    fetch(nas, nbs, 0, 0);
    mfmas((NSL - 1) & 1);
    order_copies();
  };

  // the caller issued this unit's first copies and saw them land
  fetch(L.a[0], L.b[0], 0, 0);
  // the slots line up again after P steps; the loop body is unrolled over
  // them so that every LDS address is a constant
  constexpr int P = NA == NB ? NA : NA * NB;
  int j = 0;
  for (; j + P <= KT; j += P) {
#pragma unroll
    for (int q = 0; q < P; ++q)
      step(j + q, L.a[q % NA], L.b[q % NB], L.a[(q + 1) % NA], L.b[(q + 1) % NB]);
  }
  const int rest = KT - j;  // 0..P-1 steps, starting again at slot phase 0
#pragma unroll
  for (int q = 0; q < P - 1; ++q)
    if (q < rest) step(j + q, L.a[q % NA], L.b[q % NB], L.a[(q + 1) % NA], L.b[(q + 1) % NB]);
  wait_vm<0>();  // copies past the end are still in flight
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  barrier_only();  // every wave is done with LDS
  if constexpr (STAGED) {  // the epilogue uses the ring; the next copies follow it
    store_tile_staged<BM, NW>(p, acc, ta, L);
    next();
    return;
  }
  next();  // the next unit's first copies go out before this epilogue

  if (ksp.ks > 1) {  // a K chunk of a tail tile: leave the partial to the reduction
#pragma unroll
    for (int i = 0; i < RBLK; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4)
          *part_at<RBLK, NW>(ksp.slot, (i * 4 + j) * 4 + v4) =
              make_float4(acc[i][j][4 * v4], acc[i][j][4 * v4 + 1], acc[i][j][4 * v4 + 2],
                          acc[i][j][4 * v4 + 3]);
    return;
  }
  store_tile<BM, NW, GATEUP, F8>(p, acc, ta);
}

// Unit u of an XCD's share: tile xs.tbeg + u, or (past the full rounds, when
// the tail is split) K chunk kc of tail tile q.  Every field is uniform;
// readfirstlane keeps them (and the buffer descriptors built from them) in
// SGPRs.
struct Unit {
  TileAt ta;
  KSplit ksp;
};
template <int BM>
__device__ __forceinline__ Unit unit_at(const GemmParams& p, const XcdShare& xs, int xcd, int u,
                                        int KT, int mtiles) {
  Unit w;
  int t = xs.tbeg + u;
  w.ksp = KSplit{0, KT, 1, nullptr};
  if (u >= xs.full && xs.ks > 1) {
    const int v = u - xs.full, q = v / xs.ks, kc = v - q * xs.ks;  // tail tile q, chunk kc
    t = xs.tbeg + xs.full + q;
    w.ksp.ks = xs.ks;
    w.ksp.kbeg = kc * KT / xs.ks;
    w.ksp.ksteps = (kc + 1) * KT / xs.ks - w.ksp.kbeg;
    w.ksp.slot = p.part + (size_t)(xcd * xs.nloc + v) * BM * BN;
  }
  const TileAt ta = tile_at<BM>(p, t, mtiles);
  w.ta.e = __builtin_amdgcn_readfirstlane(ta.e);
  w.ta.nt = __builtin_amdgcn_readfirstlane(ta.nt);
  w.ta.row0 = __builtin_amdgcn_readfirstlane(ta.row0);
  w.ta.nvalid = __builtin_amdgcn_readfirstlane(ta.nvalid);
  return w;
}

// Persistent grouped GEMM.  The grid holds a fixed number of workgroups (a
// multiple of 8, about one per CU); the real number of tiles is only known on
// the device (tmap[E] m-tiles x ntiles n-tiles).  Tiles are numbered in
// groups of p.gn n-tiles, m-tile major inside a group, and split into 8
// contiguous slices, one per XCD (workgroup i runs on XCD i % 8): each XCD gets
// the same share of real tiles, and the workgroups running together on one
// XCD hold neighbouring tiles, which share A row panels and weight panels in
// that XCD's L2.
// Units u, u + nloc, ... below `units` of this workgroup's share, one at a
// time: each unit's first copies go out before the previous one's epilogue.
template <int BM, int NW, bool GATEUP, bool F8, int NA, int NB, bool BT = false>
__device__ __forceinline__ void grouped_units(const GemmParams& p, const Ring& L,
                                              const XcdShare& xs, int xcd, int KT, int mtiles,
                                              int u, int units) {
  if (u >= units) return;
  const CopyPlan<BM, NW, GATEUP, F8, BT, false> cp(p.K, p.N);
  Unit cur = unit_at<BM>(p, xs, xcd, u, KT, mtiles);
  cp.template prologue<NA, NB>(tile_src<GATEUP, F8, BT>(p, cur.ta, cur.ksp), L);
  constexpr int RBLK = (2 * BM / NW) / 32;
  const int wm = cp.wave >> 1;
  for (;;) {
    wait_vm<0>();    // this unit's first copies (and the last epilogue's stores)
    barrier_only();  // ... have landed in every wave
    const int un = u + xs.nloc;
    const bool more = un < units;
    const Unit nxt = more ? unit_at<BM>(p, xs, xcd, un, KT, mtiles) : cur;
    auto next = [&]() {
      if (more) cp.template prologue<NA, NB>(tile_src<GATEUP, F8, BT>(p, nxt.ta, nxt.ksp), L);
    };
    const TileSrc src = tile_src<GATEUP, F8, BT>(p, cur.ta, cur.ksp);
    // each wave runs the fully scheduled loop over its 32-row blocks that
    // hold valid rows (rows past nvalid read zero and are not stored)
    const int act = min(RBLK, max(0, (cur.ta.nvalid - wm * (RBLK * 32) + 31) / 32));
    if (act >= RBLK)
      gemm_tile<BM, NW, GATEUP, F8, RBLK, NA, NB, BT, false, false>(p, cp, src, L, cur.ta,
                                                                    cur.ksp, next);
    else if (RBLK > 1 && act == 1)
      gemm_tile<BM, NW, GATEUP, F8, (RBLK > 1 ? 1 : 0), NA, NB, BT, false, false>(
          p, cp, src, L, cur.ta, cur.ksp, next);
    else
      gemm_tile<BM, NW, GATEUP, F8, 0, NA, NB, BT, false, false>(p, cp, src, L, cur.ta, cur.ksp,
                                                                 next);
    if (!more) break;
    u = un;
    cur = nxt;
  }
}

template <int BM, int NW, bool GATEUP, bool F8, int NA, int NB, bool BT = false>
__device__ __forceinline__ void grouped_gemm(const GemmParams& p, const Ring& L) {
  const int mtiles = p.tmap[p.E];
  const int KT = p.K / Elt<F8>::kStep;
  const int xcd = blockIdx.x & 7;
  const XcdShare xs = xcd_share(mtiles * p.ntiles, xcd, p.grid, KT, p.split_max);
  grouped_units<BM, NW, GATEUP, F8, NA, NB, BT>(p, L, xs, xcd, KT, mtiles, blockIdx.x >> 3,
                                                xs.full + xs.rem * xs.ks);
}

// LDS ring of the copy pipeline: 128-byte rows, BM-row A slots, 256-row B slots.
#define MOE_GEMM_LDS_RING                                                         \
  __shared__ __attribute__((aligned(1024))) bf16 A0[BM * BK], A1[BM * BK];        \
  __shared__ __attribute__((aligned(1024))) bf16 A2[NA == 3 ? BM * BK : 8];       \
  __shared__ __attribute__((aligned(1024))) bf16 B0[BN * BK], B1[BN * BK];        \
  __shared__ __attribute__((aligned(1024))) bf16 B2[NB == 3 ? BN * BK : 8];       \
  const Ring L{{A0, A1, A2}, {B0, B1, B2}};

// The row-grouped product with the weights stored [K][N] (input gradients:
// dA = dY W_down[e] and dX = [dG | dU] [W_gate[e]; W_up[e]]).
template <int BM, int NW, int NA, int NB>
__global__ __launch_bounds__(64 * NW) void gemm_bt_kernel(GemmParams p) {
  MOE_GEMM_LDS_RING
  grouped_gemm<BM, NW, false, false, NA, NB, true>(p, L);
}

// The gate/up GEMM on FP8 (E4M3) rows and weights with power-of-two row
// scales (GATEUP), or a plain product of them (the experts' backward: the
// output gradients' rows against W_down^T, each output scaled by its row's
// and its column's factor).
template <int BM, int NW, bool GATEUP, int NA, int NB>
__global__ __launch_bounds__(64 * NW) void gemm_fp8_kernel(GemmParams p) {
  MOE_GEMM_LDS_RING
  grouped_gemm<BM, NW, GATEUP, true, NA, NB>(p, L);
}

// Weight gradients of the expert products (section "专家计算：padding、
// block-sparse 与 grouped GEMM": the backward is a grouped product for the
// inputs and one for the weights): C_e[M][N] = sum over expert e's rows r of
// A[r][m] B[r][n], with A [rows][lda] and B [rows][ldb] the row-major
// activations (columns 0..M-1 of A, 0..N-1 of B).  Both operands are read as
// stored ([K][columns], the AT and BT copies and transposing fragment reads),
// K being expert e's rows offset[e] .. offset[e+1]-1: the buffer resources
// end at the expert's last row, so the ragged last K step reads zeros.
// Tiles (e, m-tile, n-tile) in that order (n fastest), each XCD taking a
// contiguous slice of them; the main loop is that of the row-grouped GEMM and
// the epilogue goes through LDS (store_tile_staged), after which the next
// tile's first copies go out.  An expert without rows gets one K step of
// zeros (its buffer resources are empty), i.e. C_e = 0.
__device__ __forceinline__ Unit wgrad_unit(const GemmParams& p, int t, int mt_n, int nt_n) {
  Unit w;
  const int per = mt_n * nt_n;
  const int e = t / per, r = t - e * per, mt = r / nt_n;
  w.ta.e = __builtin_amdgcn_readfirstlane(e);
  w.ta.nt = __builtin_amdgcn_readfirstlane(r - mt * nt_n);
  w.ta.row0 = __builtin_amdgcn_readfirstlane(mt * 256);  // first column m of A (row of C_e)
  w.ta.nvalid = __builtin_amdgcn_readfirstlane(min(256, p.M - mt * 256));
  const int r0 = p.offset[w.ta.e], n = p.offset[w.ta.e + 1] - r0;
  w.ksp = KSplit{__builtin_amdgcn_readfirstlane(r0),
                 __builtin_amdgcn_readfirstlane(max(1, (n + BK - 1) / BK)), 1, nullptr};
  w.ksp.ks = __builtin_amdgcn_readfirstlane(n);  // rows of the expert (0: none)
  return w;
}
__device__ __forceinline__ TileSrc wgrad_src(const GemmParams& p, const Unit& w) {
  TileSrc s;
  const size_t pa = (size_t)p.K * 2, pb = (size_t)p.Nout * 2;  // row pitches of A and B
  const size_t r0 = (size_t)w.ksp.kbeg, n = (size_t)w.ksp.ks;
  const size_t ma = (size_t)w.ta.row0 * 2, nb = (size_t)w.ta.nt * BN * 2;
  const char* A = static_cast<const char*>(p.A);
  const char* B = static_cast<const char*>(p.W0);
  s.rA = make_rsrc(A + r0 * pa + ma, n > 0 ? n * pa - ma : 0);
  s.rB0 = make_rsrc(B + r0 * pb + nb, n > 0 ? n * pb - nb : 0);
  s.rB1 = s.rB0;
  s.kbeg = 0;
  s.KT = w.ksp.ksteps;
  s.kt0 = 1 << 30;  // one panel
  // past the expert's last row both resources read zeros without touching
  // memory, so the copies past the end are left unclamped
  s.klast = 1 << 30;
  return s;
}
template <int NA, int NB>
__global__ __launch_bounds__(64 * kWaves) void gemm_wgrad_kernel(GemmParams p) {
  constexpr int BM = 256, NW = kWaves;
  MOE_GEMM_LDS_RING
  const int mt_n = (p.M + BM - 1) / BM, nt_n = (p.N + BN - 1) / BN;
  const int units = p.E * mt_n * nt_n;
  // with a grid of whole XCDs (workgroup i runs on XCD i % 8), each XCD takes
  // a contiguous slice of the tiles, so the tiles of one expert, which share
  // its row panels, run in one L2; otherwise round-robin
  int u, uend, ustep;
  if ((gridDim.x & 7) == 0) {
    const int per = (units + 7) >> 3, xcd = blockIdx.x & 7;
    u = xcd * per + (blockIdx.x >> 3);
    uend = min(units, xcd * per + per);
    ustep = gridDim.x >> 3;
  } else {
    u = blockIdx.x;
    uend = units;
    ustep = gridDim.x;
  }
  if (u >= uend) return;
  // A [rows][K = lda], B [rows][Nout = ldb]
  const CopyPlan<BM, NW, false, false, true, true> cp(0, p.Nout, p.K);
  Unit cur = wgrad_unit(p, u, mt_n, nt_n);
  cp.template prologue<NA, NB>(wgrad_src(p, cur), L);
  constexpr int RBLK = (2 * BM / NW) / 32;
  const int wm = cp.wave >> 1;
  for (;;) {
    wait_vm<0>();
    barrier_only();
    const int un = u + ustep;
    const bool more = un < uend;
    const Unit nxt = more ? wgrad_unit(p, un, mt_n, nt_n) : cur;
    auto next = [&]() {
      if (more) cp.template prologue<NA, NB>(wgrad_src(p, nxt), L);
    };
    const TileSrc src = wgrad_src(p, cur);
    // C_e is row block e of a [E * M][N] matrix (row pitch N)
    GemmParams q = p;
    q.Nout = p.N;
    Unit out = cur;
    out.ta.row0 = cur.ta.e * p.M + cur.ta.row0;
    out.ksp = KSplit{0, cur.ksp.ksteps, 1, nullptr};
    const int act = min(RBLK, max(0, (cur.ta.nvalid - wm * (RBLK * 32) + 31) / 32));
    if (act >= RBLK)
      gemm_tile<BM, NW, false, false, RBLK, NA, NB, true, true, true>(q, cp, src, L, out.ta, out.ksp,
                                                                next);
    else if (act == 1)
      gemm_tile<BM, NW, false, false, 1, NA, NB, true, true, true>(q, cp, src, L, out.ta, out.ksp,
                                                             next);
    else
      gemm_tile<BM, NW, false, false, 0, NA, NB, true, true, true>(q, cp, src, L, out.ta, out.ksp,
                                                             next);
    if (!more) break;
    u = un;
    cur = nxt;
  }
}

constexpr int kWgStores = 16;  // 2 row blocks x 4 column blocks x 2 runs of 8 columns
// A copy cursor: plain integers (uniform, kept in SGPRs); the buffer
// resources are rebuilt from them at each copy.
struct WgCursor {
  int u, j, KT;  // tile of the share, its K step, its K steps
  int r0, n;     // the expert's first row and its rows (0: none, or past the share)
  int m0, nt;    // the tile's first column of A (row of C_e) and its n-tile
  int e;         // the expert
};
__device__ __forceinline__ void wg_load(const GemmParams& p, WgCursor& c, int uend, int mt_n,
                                        int nt_n) {
  c.j = 0;
  if (c.u < uend) {
    // the same numbering as wgrad_unit; the offsets are read through the
    // constant address space, i.e. with scalar loads, which do not wait on
    // the copies and stores in flight as a vector load would
    typedef __attribute__((address_space(4))) const int32_t cint;
    const int per = mt_n * nt_n;
    const int e = c.u / per, r = c.u - e * per, mt = r / nt_n;
    cint* off = (cint*)p.offset;
    c.r0 = off[e];
    c.n = off[e + 1] - c.r0;
    c.KT = max(1, (c.n + BK - 1) / BK);
    c.m0 = mt * 256;
    c.nt = r - mt * nt_n;
    c.e = e;
  } else {  // past the share: copies from an empty resource read zeros
    c.KT = 1;
    c.r0 = c.n = c.m0 = c.nt = c.e = 0;
  }
}
// Weight gradients as one stream of K steps per workgroup.  The workgroup's
// tiles (the same XCD slices as gemm_wgrad_kernel) run their K steps back to
// back through the copy ring, A two steps ahead and B three, so the copies of
// a tile's first steps are in flight while the previous tile computes, which
// matters when experts have few rows and tiles only one or two K steps.  Each
// tile's epilogue stores straight from the accumulators with buffer stores,
// after the copies issued in its last step: every lane issues exactly
// kWgStores of them (the expert's output resource ends at its last row, and a
// column past N is sent past the resource's end), so the next step's wait
// can leave them in flight.  Vector memory loads and stores complete in issue
// order on this family: vmcnt <= BG + kWgStores there still covers every copy
// that step needs.  Requires M N 2 < 2^31 - 256 and N a multiple of 8
// (checked by the launcher).
template <int NA, int NB>
__global__ __launch_bounds__(64 * kWaves) void gemm_wgrad_stream_kernel(GemmParams p) {
  static_assert(NA == 2 && NB == 3, "ring of 2 A and 3 B slots");
  constexpr int BM = 256, NW = kWaves, WR = 2 * BM / NW, RBLK = WR / 32;
  MOE_GEMM_LDS_RING
  const int mt_n = (p.M + BM - 1) / BM, nt_n = (p.N + BN - 1) / BN;
  const int units = p.E * mt_n * nt_n;
  int u, uend, ustep;
  if ((gridDim.x & 7) == 0) {
    const int per = (units + 7) >> 3, xcd = blockIdx.x & 7;
    u = xcd * per + (blockIdx.x >> 3);
    uend = min(units, xcd * per + per);
    ustep = gridDim.x >> 3;
  } else {
    u = blockIdx.x;
    uend = units;
    ustep = gridDim.x;
  }
  if (u >= uend) return;
  using CP = CopyPlan<BM, NW, false, false, true, true>;
  constexpr int AG = CP::AG, BG = CP::BG;
  const CP cp(0, p.Nout, p.K);  // A [rows][K = lda], B [rows][Nout = ldb]
  // copy cursors: A runs two stream steps ahead of the compute, B three
  WgCursor ca, cb;
  ca.u = cb.u = u;
  wg_load(p, ca, uend, mt_n, nt_n);
  wg_load(p, cb, uend, mt_n, nt_n);
  auto advance = [&](WgCursor& c) __attribute__((always_inline)) {
    if (++c.j == c.KT) {
      c.u += ustep;
      wg_load(p, c, uend, mt_n, nt_n);
    }
  };
  // the same copies as CopyPlan::issueA / issueB over the resources of
  // wgrad_src: A [rows][K = lda] from column m0, B [rows][Nout = ldb] from
  // column BN nt, both over the expert's rows r0 .. r0 + n - 1
  auto copyA = [&](bf16* as) __attribute__((always_inline)) {
    const size_t pa = (size_t)p.K * 2, ma = (size_t)ca.m0 * 2;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(
        static_cast<const char*>(p.A) + (size_t)ca.r0 * pa + ma, ca.n > 0 ? ca.n * pa - ma : 0);
#pragma unroll
    for (int q = 0; q < AG; ++q) dma16(r, as + (cp.wave + NW * q) * 8 * BK, cp.voA[q], ca.j * cp.astep);
    advance(ca);
  };
  auto copyB = [&](bf16* bs) __attribute__((always_inline)) {
    const size_t pb = (size_t)p.Nout * 2, nb = (size_t)cb.nt * BN * 2;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(
        static_cast<const char*>(p.W0) + (size_t)cb.r0 * pb + nb, cb.n > 0 ? cb.n * pb - nb : 0);
#pragma unroll
    for (int q = 0; q < BG; ++q) dma16(r, bs + (cp.wave + NW * q) * 8 * BK, cp.voB[q], cb.j * cp.bstep);
    advance(cb);
  };
  copyA(L.a[0]);
  copyB(L.b[0]);
  copyA(L.a[1]);
  copyB(L.b[1]);
  copyB(L.b[2]);

  const int wave = cp.wave, lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1, l32 = lane & 31, khalf = lane >> 5;
  // transposing fragment reads, as in gemm_tile (AT and BT operands)
  auto tr_off = [&](int width, int x0) {
    const int l16 = lane & 15, kr = 8 * khalf + (l16 >> 2);
    const int c = (x0 + 16 * ((lane >> 4) & 1) + 4 * (l16 & 3)) >> 3;
    return kr * (width * 2) + ((c ^ trswz(kr)) * 16) + 8 * (l16 & 1);
  };
  int aoff[RBLK], boff[4];
#pragma unroll
  for (int i = 0; i < RBLK; ++i) aoff[i] = tr_off(BM, wm * WR + i * 32);
#pragma unroll
  for (int j = 0; j < 4; ++j) boff[j] = tr_off(BN, wn * 128 + j * 32);
  auto fragT = [&](const bf16* slot, int off, int slice, int width) {
    typedef short v4s __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4s lds_v4s;
    const char* q = reinterpret_cast<const char*>(slot) + off + slice * (16 * width * 2);
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(q));
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(q + 4 * width * 2));
    const v4s v[2] = {lo, hi};
    bf16x8 r;
    __builtin_memcpy(&r, v, 16);
    return r;
  };
  floatx16 acc[RBLK][4];
  auto zero = [&]() {
#pragma unroll
    for (int i = 0; i < RBLK; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  };
  zero();
  bf16x8 fa[2][RBLK], fb[2][4];
  auto fetch = [&](const bf16* as, const bf16* bs, int slice, int st) {
#pragma unroll
    for (int i = 0; i < RBLK; ++i) fa[st][i] = fragT(as, aoff[i], slice, BM);
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[st][j] = fragT(bs, boff[j], slice, BN);
  };
  auto mfmas = [&](int st) {
#pragma unroll
    for (int i = 0; i < RBLK; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[st][j], fa[st][i], acc[i][j], 0, 0, 0);
  };
  constexpr int NSL = Elt<false>::kSlices;
  constexpr int NM = RBLK * 4, NR = RBLK * 2 + 4 * 2, NC = AG + BG;
  constexpr int CPM = (NC + NM - 1) / NM, RPM = (NR + NM - 1) / NM;
  auto order = [&]() {
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (m * RPM < NR) __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);
    }
  };
  auto order_copies = [&]() {
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (m * CPM < NC) __builtin_amdgcn_sched_group_barrier(0x020, CPM, 0);
      if (m * RPM < NR) __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);
    }
  };
  // the tile being computed
  WgCursor cc;
  cc.u = u;
  wg_load(p, cc, uend, mt_n, nt_n);
  // epilogue: lane holds row l32 of each 32 x 32 block and columns
  // 8 g + 4 khalf + 0..3 (see store_tile).  The two lanes of a row swap
  // halves (v_permlane32_swap exchanges lanes 32..63 of its first operand
  // with lanes 0..31 of its second), after which lane (l32, khalf) holds
  // columns 16 h + 8 khalf + 0..7 for h = 0, 1 and stores each run of 8 as
  // one 16-byte store.  C_e is row block e of [E M][N].
  auto store = [&]() __attribute__((always_inline)) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const size_t r0 = (size_t)cc.e * p.M + cc.m0;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.C + r0 * p.N, (size_t)(p.M - cc.m0) * p.N * 2);
#pragma unroll
    for (int i = 0; i < RBLK; ++i) {
      const int rb = (wm * WR + i * 32 + l32) * p.N * 2;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const floatx16& a = acc[i][j];
          // runs g = 2 h (x) and 2 h + 1 (y) of this lane, 4 columns each
          const unsigned x0 = pack_bf16x2(a[8 * h], a[8 * h + 1]);
          const unsigned x1 = pack_bf16x2(a[8 * h + 2], a[8 * h + 3]);
          const unsigned y0 = pack_bf16x2(a[8 * h + 4], a[8 * h + 5]);
          const unsigned y1 = pack_bf16x2(a[8 * h + 6], a[8 * h + 7]);
          const auto s0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
          const u32x4 v = {s0[0], s1[0], s0[1], s1[1]};
          const int col = cc.nt * BN + wn * 128 + j * 32 + 16 * h + 8 * khalf;
          const int off = col < p.N ? rb + col * 2 : kPastEnd;
          __builtin_amdgcn_raw_buffer_store_b128(v, rc, off, 0, 0);
        }
    }
  };
  bool stored = false;  // the previous step issued a tile's stores
  // one stream step on slots (as, bs); (nas, nbs) hold the next step.  On
  // entry fa/fb[0] hold slice 0 of this step.  Returns whether work remains.
  auto step = [&](bf16* as, bf16* bs, const bf16* nas, const bf16* nbs) __attribute__((always_inline)) {
#pragma unroll
    for (int sl = 0; sl + 1 < NSL; ++sl) {
      fetch(as, bs, sl + 1, (sl + 1) & 1);
      mfmas(sl & 1);
      order();
    }
    // the next step's A and B have landed; B three steps ahead (issued
    // last) and the stores of a tile that ended at the previous step may
    // still be in flight
    if (stored) wait_vm_seen<BG + kWgStores>();
    else wait_vm_seen<BG>();
    wait_lgkm0_seen();  // this wave is done reading (as, bs)
    barrier_only();
    copyA(as);
    copyB(bs);
    fetch(nas, nbs, 0, 0);
    mfmas((NSL - 1) & 1);
    order_copies();
    stored = false;
    if (++cc.j < cc.KT) return true;
    store();
    asm volatile("" ::: "memory");
    zero();
    stored = true;
    cc.u += ustep;
    if (cc.u >= uend) return false;
    wg_load(p, cc, uend, mt_n, nt_n);
    return true;
  };
  wait_vm_seen<0>();
  barrier_only();
  fetch(L.a[0], L.b[0], 0, 0);
  // the slots line up again every 6 steps: the body is unrolled over them so
  // that every LDS address is a constant (the compiler then sees which slot
  // each copy in flight writes, and waits for none of them before reading
  // another)
  for (bool live = true; live;) {
#pragma unroll
    for (int q = 0; q < 6; ++q)
      if (live) live = step(L.a[q % 2], L.b[q % 3], L.a[(q + 1) % 2], L.b[(q + 1) % 3]);
  }
  wait_vm_seen<0>();  // copies past the share, and the last stores
}

// Epilogue of one wave's (2 BM / NW) x 128 block with 16-byte stores, the
// same number in every lane whatever the tile (rows past the tile's nvalid
// valid rows and columns past Nout fall outside the output resource and are
// dropped).  The accumulators are transposed blocks as in store_tile: lane
// holds row l32 of each 32 x 32 block and columns 8 g + 4 khalf + 0..3.  The
// two lanes of a row swap halves (v_permlane32_swap exchanges lanes 32..63 of
// its first operand with lanes 0..31 of its second), after which lane
// (l32, khalf) holds columns 16 h + 8 khalf + 0..7 of the block for h = 0, 1.
// Gate/up: a = SiLU(g) u, and with SAVE also g and u into C2.  Stores per
// lane: RBLK * (GATEUP ? 2 : 4) * 2, three times that with SAVE.
template <int BM, int NW, bool GATEUP, bool SAVE, bool F8 = false>
__device__ __forceinline__ void store_tile16(const GemmParams& p,
                                             const floatx16 (&acc)[(2 * BM / NW) / 32][4],
                                             int row0, int nvalid, int nt, int wave, int lane,
                                             int e = 0) {
  constexpr int WR = 2 * BM / NW, RBLK = WR / 32;
  const int wm = wave >> 1, wn = wave & 1, l32 = lane & 31, khalf = lane >> 5;
  auto pack8 = [&](const float* x, const float* y) __attribute__((always_inline)) {
    const auto s0 = __builtin_amdgcn_permlane32_swap(pack_bf16x2(x[0], x[1]),
                                                     pack_bf16x2(y[0], y[1]), false, false);
    const auto s1 = __builtin_amdgcn_permlane32_swap(pack_bf16x2(x[2], x[3]),
                                                     pack_bf16x2(y[2], y[3]), false, false);
    const u32x4 v = {s0[0], s1[0], s0[1], s1[1]};
    return v;
  };
  const int pitch = p.Nout * 2;
  const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.C + (size_t)row0 * p.Nout, (size_t)nvalid * pitch);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(SAVE ? p.C2 + (size_t)row0 * 2 * p.Nout : p.C,
                                              SAVE ? (size_t)nvalid * 2 * pitch : 0);
#pragma unroll
  for (int i = 0; i < RBLK; ++i) {
    const int r = wm * WR + i * 32 + l32;
    // FP8: the row's power-of-two scale (rows past the valid ones, never
    // stored, take the last valid row's)
    const float sa = F8 ? p.sa[row0 + min(r, nvalid - 1)] : 1.f;
#pragma unroll
    for (int j = 0; j < (GATEUP ? 2 : 4); ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int col = (GATEUP ? nt * 128 + wn * 64 : nt * BN + wn * 128) + j * 32 + 16 * h +
                        8 * khalf;
        const bool in = col < p.Nout;
        // runs 2 h (x) and 2 h + 1 (y) of this lane's own columns (before
        // the swap): they start at cx and cx + 8
        const int cx = (GATEUP ? nt * 128 + wn * 64 : nt * BN + wn * 128) + j * 32 + 16 * h +
                       4 * khalf;
        float sgx[4] = {1.f, 1.f, 1.f, 1.f}, sgy[4] = {1.f, 1.f, 1.f, 1.f};
        float sux[4] = {1.f, 1.f, 1.f, 1.f}, suy[4] = {1.f, 1.f, 1.f, 1.f};
        if (F8) {  // power-of-two scales: the products are exact
          const size_t b = (size_t)e * p.N;
          const int c0 = cx < p.Nout ? cx : 0, c1 = cx + 8 < p.Nout ? cx + 8 : 0;
          const float4 a0 = *reinterpret_cast<const float4*>(p.sw0 + b + c0);
          const float4 a1 = *reinterpret_cast<const float4*>(p.sw0 + b + c1);
          sgx[0] = sa * a0.x; sgx[1] = sa * a0.y; sgx[2] = sa * a0.z; sgx[3] = sa * a0.w;
          sgy[0] = sa * a1.x; sgy[1] = sa * a1.y; sgy[2] = sa * a1.z; sgy[3] = sa * a1.w;
          if (GATEUP) {
            const float4 b0 = *reinterpret_cast<const float4*>(p.sw1 + b + c0);
            const float4 b1 = *reinterpret_cast<const float4*>(p.sw1 + b + c1);
            sux[0] = sa * b0.x; sux[1] = sa * b0.y; sux[2] = sa * b0.z; sux[3] = sa * b0.w;
            suy[0] = sa * b1.x; suy[1] = sa * b1.y; suy[2] = sa * b1.z; suy[3] = sa * b1.w;
          }
        }
        float x[4], y[4], gx[4], gy[4], ux[4], uy[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          gx[t] = acc[i][j][8 * h + t] * sgx[t];
          gy[t] = acc[i][j][8 * h + 4 + t] * sgy[t];
          if (GATEUP) {  // SiLU(g) u with the hardware reciprocal, as in store_tile
            ux[t] = acc[i][j + 2][8 * h + t] * sux[t];
            uy[t] = acc[i][j + 2][8 * h + 4 + t] * suy[t];
            x[t] = gx[t] * ux[t] * __builtin_amdgcn_rcpf(1.f + __expf(-gx[t]));
            y[t] = gy[t] * uy[t] * __builtin_amdgcn_rcpf(1.f + __expf(-gy[t]));
          } else {
            x[t] = gx[t];
            y[t] = gy[t];
          }
        }
        __builtin_amdgcn_raw_buffer_store_b128(pack8(x, y), rc, in ? r * pitch + col * 2 : kPastEnd,
                                               0, 0);
        if (SAVE) {
          const int ro = r * 2 * pitch;
          __builtin_amdgcn_raw_buffer_store_b128(pack8(gx, gy), rs, in ? ro + col * 2 : kPastEnd,
                                                 0, 0);
          __builtin_amdgcn_raw_buffer_store_b128(pack8(ux, uy), rs,
                                                 in ? ro + pitch + col * 2 : kPastEnd, 0, 0);
        }
      }
  }
}

// Forward grouped GEMM with the copy ring running across units (bf16).  The
// workgroup's units are those of grouped_gemm (the same XCD slices, rounds
// and K chunks of a split tail round), one at a time as there, but the copies
// that would run past a unit's last K step fetch the next unit's first steps
// instead: the next unit starts with its first NA + NB stages already in
// flight, no wave waits for the ring to drain between units, and the
// epilogue's stores overlap those copies.  The ring's slots therefore start a
// unit at the phase where the previous one left them: unit i starts at slot
// phase (sum of the earlier units' K steps) mod P.  Each unit's steps run with
// its slots rotated to phase 0 and passed as restrict parameters, together
// with the operands: the compiler then tags each copy (its buffer resource is
// based on an operand parameter) and each fragment read with its slot, and
// its own wait insertion makes a read wait only for copies into that slot.
//
// Epilogue: straight from the accumulators after the unit's last copies, with
// the same number of stores in every lane whatever the unit (rows past the
// unit's valid rows and columns past Nout fall outside the output resource
// and are dropped), so that the next unit's first wait can leave exactly
// those stores and the newest copies in flight (vector memory operations
// complete in issue order on this family).
struct FwUnit {
  int u;                          // unit of the workgroup's share
  int kbeg, KT, ks;               // first K step, K steps, K chunks of the tile (1: whole)
  int e, nt, row0, nvalid, live;  // the tile (live = 0: past the share)
};
__device__ __forceinline__ FwUnit fw_unit(const GemmParams& p, const XcdShare& xs, int units,
                                          int mtiles, int KT, int u) {
  typedef __attribute__((address_space(4))) const int32_t cint;
  FwUnit c;
  c.u = u;
  c.kbeg = 0;
  c.KT = KT;
  c.ks = 1;
  c.e = c.nt = c.row0 = c.nvalid = c.live = 0;
  if (u >= units) return c;  // copies from empty resources read zeros
  int t = xs.tbeg + u;
  if (u >= xs.full && xs.ks > 1) {  // K chunk kc of tail tile q (as unit_at)
    const int v = u - xs.full, q = v / xs.ks, kc = v - q * xs.ks;
    t = xs.tbeg + xs.full + q;
    c.ks = xs.ks;
    c.kbeg = kc * KT / xs.ks;
    c.KT = (kc + 1) * KT / xs.ks - c.kbeg;
  }
  // tile t of the numbering of tile_at, read with scalar loads
  const int g = t / (mtiles * p.gn);
  const int r = t - g * mtiles * p.gn;
  const int gw = min(p.gn, p.ntiles - g * p.gn);
  const int mt = r / gw;
  const cint* tab = (cint*)p.tmap + ((p.E + 2) & ~1);
  const int m0 = tab[2 * mt], m1 = tab[2 * mt + 1];
  c.nt = g * p.gn + r % gw;
  c.e = m1 & 0xffff;
  c.row0 = m0;
  c.nvalid = m1 >> 16;
  c.live = 1;
  return c;
}

// CFIRST: each step's copies are all issued right after the barrier, ahead of
// the last slice's MFMAs, instead of one per MFMA (weight-streaming shapes,
// where every expert fits one m-tile: the copies then start earlier; on
// MFMA-bound shapes the burst slows the slice down).
template <int BM, int NA, int NB, bool GATEUP, bool SAVE, bool F8 = false, bool CFIRST = false>
__global__ __launch_bounds__(64 * kWaves) void gemm_chain_kernel(GemmParams p) {
  constexpr int NW = kWaves, WR = 2 * BM / NW, RBLK = WR / 32;
  constexpr int P = NA == NB ? NA : NA * NB;  // the slots line up again after P steps
  static_assert(RBLK >= 1 && (NA == 2 || NA == 3) && NB == 3, "ring");
  static_assert(GATEUP || !SAVE, "pre-activations are a gate/up output");
  MOE_GEMM_LDS_RING
  typedef __attribute__((address_space(4))) const int32_t cint;
  const int mtiles = ((cint*)p.tmap)[p.E];
  const int KT = p.K / Elt<F8>::kStep;
  const int xcd = blockIdx.x & 7;
  const XcdShare xs = xcd_share(mtiles * p.ntiles, xcd, p.grid, KT, p.split_max);
  const int units = xs.full + xs.rem * xs.ks;
  if ((int)(blockIdx.x >> 3) >= units) return;
  using CP = CopyPlan<BM, NW, GATEUP, F8>;
  constexpr int AG = CP::AG, BG = CP::BG;
  const CP cp(p.K, p.N);
  const int wave = cp.wave, lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1, l32 = lane & 31, khalf = lane >> 5;
  const int sw = (l32 >> 1) & 7;  // (row >> 1) & 7 of every fragment row of this lane
  const size_t rb = (size_t)p.K * Elt<F8>::kBytes;  // bytes per row of A and of the weights
  constexpr int FC = F8 ? 2 : 1;  // 16-byte chunks per fragment and lane
  using Frag = typename Elt<F8>::Frag;
  int aoff[RBLK], boff[4];
#pragma unroll
  for (int i = 0; i < RBLK; ++i) aoff[i] = (wm * WR + i * 32 + l32) * 128;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = GATEUP ? ((j < 2 ? 0 : 128) + wn * 64 + (j & 1) * 32 + l32)
                         : (wn * 128 + j * 32 + l32);
    boff[j] = r * 128;
  }
  Frag fa[2][RBLK], fb[2][4];
  // one fragment: FC chunks of 16 bytes of a row, at physical chunks c ^ sw
  auto frag = [&](const bf16* slot, int off, int c0) __attribute__((always_inline)) {
    const char* row = reinterpret_cast<const char*>(slot) + off;
    if constexpr (F8) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(row + ((c0 ^ sw) * 16));
      const u32x4 y = *reinterpret_cast<const u32x4*>(row + (((c0 + 1) ^ sw) * 16));
      return Frag{(int)x[0], (int)x[1], (int)x[2], (int)x[3],
                  (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
    } else {
      return *reinterpret_cast<const Frag*>(row + ((c0 ^ sw) * 16));
    }
  };
  // all the fragments of a slice (the next unit's slice 0 is read whatever
  // its rows)
  auto fetch = [&](const bf16* as, const bf16* bs, int slice, int st) __attribute__((always_inline)) {
    const int c0 = FC * (2 * slice + khalf);
#pragma unroll
    for (int i = 0; i < RBLK; ++i) fa[st][i] = frag(as, aoff[i], c0);
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[st][j] = frag(bs, boff[j], c0);
  };
  // buffer resources of a unit's A rows and weight panels
  auto srcA = [&](const char* Ag, const FwUnit& c) __attribute__((always_inline)) {
    return make_rsrc(Ag + (size_t)c.row0 * rb, (size_t)c.nvalid * rb);
  };
  auto srcB = [&](const char* W, const FwUnit& c) __attribute__((always_inline)) {
    const size_t n0 = (size_t)c.nt * (GATEUP ? 128 : BN);
    return make_rsrc(W + ((size_t)c.e * p.N + n0) * rb, c.live ? (size_t)(p.N - n0) * rb : 0);
  };
  auto copyA = [&](__amdgpu_buffer_rsrc_t r, bf16* as, int kb) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < AG; ++q) dma16(r, as + (wave + NW * q) * 8 * BK, cp.voA[q], kb);
  };
  auto copyB = [&](__amdgpu_buffer_rsrc_t r0, __amdgpu_buffer_rsrc_t r1, bf16* bs, int kb)
                   __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < BG; ++q)
      dma16((GATEUP && q >= BG / 2) ? r1 : r0, bs + (wave + NW * q) * 8 * BK, cp.voB[q], kb);
  };

  constexpr int NSL = Elt<F8>::kSlices;
  constexpr int kWaitBase = BG + (NA == 3 ? AG : 0);
  const char* const pA = static_cast<const char*>(p.A);
  const char* const pW0 = static_cast<const char*>(p.W0);
  const char* const pW1 = static_cast<const char*>(p.W1 ? p.W1 : p.W0);

  // One unit: its K steps on slots rotated so that its step 0 is in a0 / b0.
  // On entry fa/fb[0] hold slice 0 of step 0, and the copies of the unit's
  // steps 0 .. NA-1 (A) and 0 .. NB-1 (B) are in flight, followed by the
  // previous unit's epilogue stores.  R: this wave's 32-row
  // blocks with valid rows (RBLK or none: a wave with some valid rows runs
  // all its blocks).
  auto unit = [&](auto Rc, bf16* __restrict__ a0, bf16* __restrict__ a1, bf16* __restrict__ a2,
                  bf16* __restrict__ b0, bf16* __restrict__ b1, bf16* __restrict__ b2,
                  const char* __restrict__ Ag, const char* __restrict__ Wg,
                  const char* __restrict__ Wu, const FwUnit& cur, const FwUnit& nxt)
                  __attribute__((always_inline)) {
    constexpr int R = decltype(Rc)::value;
    bf16* const A[3] = {a0, a1, a2};
    bf16* const B[3] = {b0, b1, b2};
    const __amdgpu_buffer_rsrc_t rA = srcA(Ag, cur), rB0 = srcB(Wg, cur), rB1 = srcB(Wu, cur);
    const __amdgpu_buffer_rsrc_t nA = srcA(Ag, nxt), nB0 = srcB(Wg, nxt), nB1 = srcB(Wu, nxt);
    const int KTu = cur.KT;
    floatx16 acc[RBLK][4];
#pragma unroll
    for (int i = 0; i < RBLK; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
    auto mfmas = [&](int st) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < R; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if constexpr (F8)  // format codes 0, 0: both operands E4M3; no block scales
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                fb[st][j], fa[st][i], acc[i][j], 0, 0, 0, 0, 0, 0);
          else
            acc[i][j] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[st][j], fa[st][i], acc[i][j], 0, 0, 0);
    };
    constexpr int NM = R * 4, NR = (RBLK + 4) * FC, NC = AG + BG;
    constexpr int CPM = NM > 0 ? (NC + NM - 1) / NM : NC, RPM = NM > 0 ? (NR + NM - 1) / NM : NR;
    auto order = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (m * RPM < NR) __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);
      }
    };
    auto order_copies = [&]() __attribute__((always_inline)) {
      if constexpr (CFIRST) __builtin_amdgcn_sched_group_barrier(0x020, NC, 0);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (!CFIRST && m * CPM < NC) __builtin_amdgcn_sched_group_barrier(0x020, CPM, 0);
        if (m * RPM < NR) __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);
      }
    };
    // step j on slots (as, bs); (nas, nbs) hold step j + 1 (or the next
    // unit's step 0)
    auto step = [&](int j, bf16* as, bf16* bs, const bf16* nas, const bf16* nbs)
                    __attribute__((always_inline)) {
      if (R > 0) {
#pragma unroll
        for (int sl = 0; sl + 1 < NSL; ++sl) {
          fetch(as, bs, sl + 1, (sl + 1) & 1);
          mfmas(sl & 1);
          order();
        }
      }
      // step j + 1's A and B have landed; the copies issued in the previous
      // step for later steps may still be in flight (at a unit's step 0 this
      // also retires the previous unit's epilogue stores and its last B
      // copies: one early wait per unit, for one wait count that the
      // compiler's own wait insertion can follow everywhere)
      wait_vm_seen<kWaitBase>();
      wait_lgkm0_seen();  // this wave is done reading (as, bs)
      barrier_only();
      // into the slots just read: A for step j + NA and B for step j + NB,
      // of this unit or, past its end, of the next one
      const int sa = j + NA, sb = j + NB;
      const bool na = sa >= KTu, nb = sb >= KTu;
      const __amdgpu_buffer_rsrc_t ra = na ? nA : rA;
      const __amdgpu_buffer_rsrc_t rb0 = nb ? nB0 : rB0, rb1 = nb ? nB1 : rB1;
      const int ka = (na ? nxt.kbeg + sa - KTu : cur.kbeg + sa) * 128;
      const int kb = (nb ? nxt.kbeg + sb - KTu : cur.kbeg + sb) * 128;
      if (NA == 2) copyA(ra, as, ka);
      copyB(rb0, rb1, bs, kb);
      if (NA == 3) copyA(ra, as, ka);
      fetch(nas, nbs, 0, 0);
      if (R > 0) {
        mfmas((NSL - 1) & 1);
        order_copies();
      } else {  // the fragment reads before this step's copies
        __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, NC, 0);
      }
    };
    int j = 0;
    for (; j + P <= KTu; j += P) {
#pragma unroll
      for (int q = 0; q < P; ++q)
        step(j + q, A[q % NA], B[q % NB], A[(q + 1) % NA], B[(q + 1) % NB]);
    }
    const int rest = KTu - j;  // 0 .. P-1 steps, starting again at slot phase 0
#pragma unroll
    for (int q = 0; q < P - 1; ++q)
      if (q < rest) step(j + q, A[q % NA], B[q % NB], A[(q + 1) % NA], B[(q + 1) % NB]);

    // epilogue
    if (cur.ks > 1) {  // a K chunk of a tail tile: its float32 partial
      float* slot = p.part + (size_t)(xcd * xs.nloc + (cur.u - xs.full)) * BM * BN;
#pragma unroll
      for (int i = 0; i < RBLK; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4)
            *part_at<RBLK, NW>(slot, (i * 4 + jj) * 4 + v4) =
                make_float4(acc[i][jj][4 * v4], acc[i][jj][4 * v4 + 1], acc[i][jj][4 * v4 + 2],
                            acc[i][jj][4 * v4 + 3]);
      return;
    }
    store_tile16<BM, NW, GATEUP, SAVE, F8>(p, acc, cur.row0, cur.nvalid, cur.nt, wave, lane, cur.e);
  };
  // the first unit's first copies, into slot phase 0 (its own restrict scope)
  FwUnit cur = fw_unit(p, xs, units, mtiles, KT, blockIdx.x >> 3);
  auto prologue = [&](bf16* __restrict__ a0, bf16* __restrict__ a1, bf16* __restrict__ a2,
                      bf16* __restrict__ b0, bf16* __restrict__ b1, bf16* __restrict__ b2,
                      const char* __restrict__ Ag, const char* __restrict__ Wg,
                      const char* __restrict__ Wu) __attribute__((always_inline)) {
    // steps past a short unit's end copy its last step again (in bounds,
    // never read): the next unit then starts from a full prologue
    const __amdgpu_buffer_rsrc_t rA = srcA(Ag, cur), rB0 = srcB(Wg, cur), rB1 = srcB(Wu, cur);
    bf16* const A[3] = {a0, a1, a2};
    bf16* const B[3] = {b0, b1, b2};
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      const int k = (cur.kbeg + min(s, cur.KT - 1)) * 128;
      if (s < NA) copyA(rA, A[s], k);
      copyB(rB0, rB1, B[s], k);
    }
    wait_vm_seen<0>();
    barrier_only();
    fetch(a0, b0, 0, 0);
  };
  // (with 2 A slots the third A parameter repeats slot 0 and is never used)
  prologue(L.a[0], L.a[1], L.a[NA == 3 ? 2 : 0], L.b[0], L.b[1], L.b[2], pA, pW0, pW1);
  int ph = 0;
  for (;;) {
    const FwUnit nxt = fw_unit(p, xs, units, mtiles, KT, cur.u + xs.nloc);
    // rotate the slots so that this unit's step 0 is in slot 0 (selects
    // among the slots, so that only the ring's own slots are referenced)
    auto rotA = [&](int k) __attribute__((always_inline)) {
      if (NA == 2) return (k & 1) ? L.a[1] : L.a[0];
      const int m = k % 3;
      return m == 0 ? L.a[0] : (m == 1 ? L.a[1] : L.a[2]);
    };
    auto rotB = [&](int k) __attribute__((always_inline)) {
      const int m = k % 3;
      return m == 0 ? L.b[0] : (m == 1 ? L.b[1] : L.b[2]);
    };
    bf16* const A0 = rotA(ph);
    bf16* const A1 = rotA(ph + 1);
    bf16* const A2 = rotA(ph + 2);
    bf16* const B0r = rotB(ph);
    bf16* const B1r = rotB(ph + 1);
    bf16* const B2r = rotB(ph + 2);
    if (wm * WR < cur.nvalid)
      unit(std::integral_constant<int, RBLK>{}, A0, A1, A2, B0r, B1r, B2r, pA, pW0, pW1, cur,
           nxt);
    else
      unit(std::integral_constant<int, 0>{}, A0, A1, A2, B0r, B1r, B2r, pA, pW0, pW1, cur, nxt);
    if (!nxt.live) break;
    ph = (ph + cur.KT) % P;
    cur = nxt;
  }
  wait_vm_seen<0>();  // copies past the share, and the last stores
}

// Sum of the K chunks of the tail tiles, in chunk order, then the same
// epilogue as the GEMM kernels.  Workgroup b handles tail tile b / 8 of XCD
// b % 8 (if that XCD split its tail); thread i reads the partial groups that
// thread i of the GEMM wrote.
template <int BM, int NW, bool GATEUP, bool F8>
__global__ __launch_bounds__(64 * NW) void ksplit_reduce_kernel(GemmParams p) {
  constexpr int RBLK = (2 * BM / NW) / 32;
  const int mtiles = p.tmap[p.E];
  const int xcd = blockIdx.x & 7, q = blockIdx.x >> 3;
  const XcdShare xs =
      xcd_share(mtiles * p.ntiles, xcd, p.grid, p.K / Elt<F8>::kStep, p.split_max);
  if (xs.ks <= 1 || q >= xs.rem) return;
  const TileAt ta = tile_at<BM>(p, xs.tbeg + xs.full + q, mtiles);
  floatx16 acc[RBLK][4];
#pragma unroll
  for (int i = 0; i < RBLK; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  for (int c = 0; c < xs.ks; ++c) {
    float* slot = p.part + (size_t)(xcd * xs.nloc + q * xs.ks + c) * BM * BN;
#pragma unroll
    for (int i = 0; i < RBLK; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          const float4 x = *part_at<RBLK, NW>(slot, (i * 4 + j) * 4 + v4);
          acc[i][j][4 * v4] += x.x;
          acc[i][j][4 * v4 + 1] += x.y;
          acc[i][j][4 * v4 + 2] += x.z;
          acc[i][j][4 * v4 + 3] += x.w;
        }
  }
  store_tile<BM, NW, GATEUP, F8>(p, acc, ta);
}

// The same sum for bf16 outputs, by wave rows: workgroup b (two waves) takes
// wave row (b / 8) % 4 of tail tile b / 32 of XCD b % 8, i.e. the partials of
// the GEMM's waves 2 wm and 2 wm + 1, and stores them with store_tile16.  Four
// workgroups per tile keep more loads in flight than one.
template <int BM, bool GATEUP, bool SAVE>
__global__ __launch_bounds__(128) void ksplit_sum_kernel(GemmParams p) {
  constexpr int NW = kWaves, RBLK = (2 * BM / NW) / 32;
  const int mtiles = p.tmap[p.E];
  const int xcd = blockIdx.x & 7, rest = blockIdx.x >> 3, q = rest >> 2, wm = rest & 3;
  const XcdShare xs = xcd_share(mtiles * p.ntiles, xcd, p.grid, p.K / BK, p.split_max);
  if (xs.ks <= 1 || q >= xs.rem) return;
  const TileAt ta = tile_at<BM>(p, xs.tbeg + xs.full + q, mtiles);
  const int wave = 2 * wm + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int tid = wave * 64 + lane;  // the GEMM thread that wrote these partials
  floatx16 acc[RBLK][4];
#pragma unroll
  for (int i = 0; i < RBLK; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  for (int c = 0; c < xs.ks; ++c) {  // in chunk order
    const float4* slot =
        reinterpret_cast<const float4*>(p.part + (size_t)(xcd * xs.nloc + q * xs.ks + c) * BM * BN);
#pragma unroll
    for (int i = 0; i < RBLK; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          const float4 x = slot[(size_t)((i * 4 + j) * 4 + v4) * 64 * NW + tid];
          acc[i][j][4 * v4] += x.x;
          acc[i][j][4 * v4 + 1] += x.y;
          acc[i][j][4 * v4 + 2] += x.z;
          acc[i][j][4 * v4 + 3] += x.w;
        }
  }
  store_tile16<BM, NW, GATEUP, SAVE>(p, acc, ta.row0, ta.nvalid, ta.nt, wave, lane);
}

// float32 path: one thread per output, plain dot products (small workloads).
template <bool GATEUP>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* A, const int32_t* offset,
                                                       const float* W0, const float* W1,
                                                       float* C, int E, int K, int N) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int rows = offset[E];
  if (i >= (int64_t)rows * N) return;
  const int row = (int)(i / N), col = (int)(i % N);
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offset[mid] <= row) lo = mid; else hi = mid;
  }
  // 16-byte loads (K is a multiple of 4): each lane's weight row is read four
  // elements per load, the products still added in k order
  const float4* a = reinterpret_cast<const float4*>(A + (size_t)row * K);
  const float4* w0 = reinterpret_cast<const float4*>(W0 + ((size_t)lo * N + col) * K);
  float s0 = 0.f;
  if (GATEUP) {
    const float4* w1 = reinterpret_cast<const float4*>(W1 + ((size_t)lo * N + col) * K);
    float s1 = 0.f;
    for (int j = 0; j < K / 4; ++j) {
      const float4 x = a[j], g = w0[j], u = w1[j];
      s0 = fmaf(x.w, g.w, fmaf(x.z, g.z, fmaf(x.y, g.y, fmaf(x.x, g.x, s0))));
      s1 = fmaf(x.w, u.w, fmaf(x.z, u.z, fmaf(x.y, u.y, fmaf(x.x, u.x, s1))));
    }
    C[i] = s0 / (1.f + expf(-s0)) * s1;
  } else {
    for (int j = 0; j < K / 4; ++j) {
      const float4 x = a[j], g = w0[j];
      s0 = fmaf(x.w, g.w, fmaf(x.z, g.z, fmaf(x.y, g.y, fmaf(x.x, g.x, s0))));
    }
    C[i] = s0;
  }
}

// Tile maps of both GEMMs' row tiles (see tile_maps_block) from the offsets.
__global__ __launch_bounds__(256) void tile_map_kernel(const int32_t* offset, int E, int bm1,
                                                       int bm2, int32_t* m1, int32_t* m2) {
  __shared__ int tmp[8];
  const int e = threadIdx.x;
  const int n = e < E ? offset[e + 1] - offset[e] : 0;
  tile_maps_block(e, E, n, e < E ? offset[e] : 0, bm1, bm2, m1, m2, tmp);
}

// Offsets of a dense pass over all T rows as one "expert" (the shared
// experts): {0, T}.
__global__ void dense_offsets_kernel(int T, int32_t* offset) {
  if (threadIdx.x == 0) {
    offset[0] = 0;
    offset[1] = T;
  }
}

int round8(int x) { return (x + 7) & ~7; }

// Copy pipelines (LDS slots of A and B tiles): weight tiles go 3 steps ahead
// (they come from HBM, or from L2 behind other workgroups' misses), A tiles 2
// steps ahead in 256-row tiles (2 x 32 KB + 3 x 32 KB fill the 160 KB of LDS)
// and 3 in 128-row tiles.
// cfirst: the weight-streaming schedule of the copies (256-row tiles without
// the pre-activation output).
template <bool GATEUP>
void launch_gemm(int bm, const GemmParams& p, hipStream_t s, bool cfirst = false) {
  const dim3 grid(p.grid), block(64 * kWaves);
  const bool save = GATEUP && p.C2;
  if (bm == 256) {
    if (save)
      hipLaunchKernelGGL((gemm_chain_kernel<256, 2, 3, GATEUP, GATEUP>), grid, block, 0, s, p);
    else if (cfirst)
      hipLaunchKernelGGL((gemm_chain_kernel<256, 2, 3, GATEUP, false, false, true>), grid, block,
                         0, s, p);
    else
      hipLaunchKernelGGL((gemm_chain_kernel<256, 2, 3, GATEUP, false>), grid, block, 0, s, p);
    if (save)
      hipLaunchKernelGGL((ksplit_sum_kernel<256, GATEUP, GATEUP>), dim3(4 * p.grid), dim3(128), 0,
                         s, p);
    else
      hipLaunchKernelGGL((ksplit_sum_kernel<256, GATEUP, false>), dim3(4 * p.grid), dim3(128), 0,
                         s, p);
  } else {
    if (save)
      hipLaunchKernelGGL((gemm_chain_kernel<128, 3, 3, GATEUP, GATEUP>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((gemm_chain_kernel<128, 3, 3, GATEUP, false>), grid, block, 0, s, p);
    if (save)
      hipLaunchKernelGGL((ksplit_sum_kernel<128, GATEUP, GATEUP>), dim3(4 * p.grid), dim3(128), 0,
                         s, p);
    else
      hipLaunchKernelGGL((ksplit_sum_kernel<128, GATEUP, false>), dim3(4 * p.grid), dim3(128), 0,
                         s, p);
  }
}

void launch_gemm_bt(int bm, const GemmParams& p, hipStream_t s) {
  const dim3 grid(p.grid), block(64 * kWaves);
  if (bm == 256) {
    hipLaunchKernelGGL((gemm_bt_kernel<256, kWaves, 2, 3>), grid, block, 0, s, p);
    hipLaunchKernelGGL((ksplit_sum_kernel<256, false, false>), dim3(4 * p.grid), dim3(128), 0, s,
                       p);
  } else {
    hipLaunchKernelGGL((gemm_bt_kernel<128, kWaves, 3, 3>), grid, block, 0, s, p);
    hipLaunchKernelGGL((ksplit_sum_kernel<128, false, false>), dim3(4 * p.grid), dim3(128), 0, s,
                       p);
  }
}

template <bool GATEUP>
void launch_gemm_fp8(int bm, const GemmParams& p, hipStream_t s) {
  const dim3 grid(p.grid), block(64 * kWaves);
  if (bm == 256) {
    hipLaunchKernelGGL((gemm_chain_kernel<256, 2, 3, GATEUP, false, true>), grid, block, 0, s, p);
    hipLaunchKernelGGL((ksplit_reduce_kernel<256, kWaves, GATEUP, true>), grid, block, 0, s, p);
  } else {
    hipLaunchKernelGGL((gemm_chain_kernel<128, 3, 3, GATEUP, false, true>), grid, block, 0, s, p);
    hipLaunchKernelGGL((ksplit_reduce_kernel<128, kWaves, GATEUP, true>), grid, block, 0, s, p);
  }
}

}  // namespace

FfnShape ffn_shape(int64_t rows_max, int E, int h, int f, int T, int k, int bf16_, int ncu) {
  FfnShape fs{};
  if (!bf16_) {
    fs.bm1 = fs.bm2 = 1;
    return fs;
  }
  // 256-row tiles unless the average expert has at most 96 rows.  With 8
  // waves (4 along M x 2 along N) waves w and w + 4 share a SIMD, so the first
  // two wave rows already cover all four SIMDs: a tile of an expert with
  // 100-200 rows wastes little, and each expert's weights are streamed once
  // per n-tile instead of once per 128-row tile.
  const double avg = E > 0 ? (double)T * k / E : 0.0;
  fs.bm1 = fs.bm2 = avg <= 96.0 ? 128 : 256;
  fs.nw1 = fs.nw2 = kWaves;
  fs.mt1 = (int)((rows_max + (int64_t)E * (fs.bm1 - 1)) / fs.bm1);
  fs.mt2 = (int)((rows_max + (int64_t)E * (fs.bm2 - 1)) / fs.bm2);
  fs.nt1 = (f + 127) / 128;
  fs.nt2 = (h + BN - 1) / BN;
  fs.rows_cap = (int)rows_max;
  // persistent grid: one workgroup per CU (the LDS pipeline takes most of a
  // CU), never more than the static bound on tiles, a multiple of 8
  fs.grid1 = round8(std::min<int64_t>((int64_t)fs.mt1 * fs.nt1, ncu));
  fs.grid2 = round8(std::min<int64_t>((int64_t)fs.mt2 * fs.nt2, ncu));
  // tail tiles are cut into at most 4 K chunks: each chunk's float32
  // partial (256 KB) is written and read back once by the reduction
  fs.split_max = 4;
  fs.part_slots = std::max(fs.grid1, fs.grid2);
  // Groups of 8 n-tiles, except for the down product of experts that fit
  // one m-tile: there each weight panel is read once anyway, and a group of
  // (up to 32) n-tiles reads an expert's A panel from the fabric once instead
  // of once per group (DeepSeek-V3 shape, 28 n-tiles: down 4.8% faster; the
  // gate/up product measured 0.6% slower with wide groups).
  fs.gn1 = fs.gn2 = GN;
  if (avg <= (double)fs.bm2) fs.gn2 = std::min(fs.nt2, 32);
  // Experts that fit one m-tile read each weight byte once: the products are
  // bound by that stream, and issuing each step's copies in one burst helps
  // it (DeepSeek-V3 shape: gate/up 2.92 -> 2.86 ms, down 1.63 -> 1.61 ms; the
  // Mixtral and noisy shapes ran 1.5-2.4% slower with it).
  fs.wstream = avg <= (double)fs.bm2 ? 1 : 0;
  return fs;
}

hipError_t launch_tile_map(const int32_t* offset, int E, int bm1, int bm2, int32_t* map1,
                           int32_t* map2, hipStream_t s) {
  hipLaunchKernelGGL(tile_map_kernel, dim3(1), dim3(256), 0, s, offset, E, bm1, bm2, map1, map2);
  return hipGetLastError();
}

hipError_t launch_dense_offsets(int T, int32_t* offset, hipStream_t s) {
  hipLaunchKernelGGL(dense_offsets_kernel, dim3(1), dim3(64), 0, s, T, offset);
  return hipGetLastError();
}

hipError_t launch_gate_up(const FfnShape& fs, const void* X, const int32_t* offset,
                          const int32_t* map1, const void* Wg, const void* Wu, void* A,
                          float* part, int E, int h, int f, int bf16_, hipStream_t s) {
  if (!bf16_) {
    // rows are bounded by the caller's rows_max; launch for the static bound
    return hipErrorNotSupported;
  }
  if (fs.grid1 == 0) return hipSuccess;
  GemmParams p{X, offset, map1, Wg, Wu, static_cast<bf16*>(A), nullptr, nullptr, nullptr,
               E, h, f, f, fs.nt1, fs.mt1, part, fs.split_max, fs.grid1};
  p.gn = fs.gn1;
  launch_gemm<true>(fs.bm1, p, s, fs.wstream);
  return hipGetLastError();
}

hipError_t launch_gate_up_fp8(const FfnShape& fs, const void* X8, const float* x_scale,
                              const int32_t* offset, const int32_t* map1, const void* Wg8,
                              const float* s_gate, const void* Wu8, const float* s_up, void* A,
                              float* part, int E, int h, int f, hipStream_t s) {
  if (fs.grid1 == 0) return hipSuccess;
  GemmParams p{X8, offset, map1, Wg8, Wu8, static_cast<bf16*>(A), x_scale, s_gate, s_up,
               E, h, f, f, fs.nt1, fs.mt1, part, fs.split_max, fs.grid1};
  p.gn = fs.gn1;
  launch_gemm_fp8<true>(fs.bm1, p, s);
  return hipGetLastError();
}

hipError_t launch_gate_up_save(const FfnShape& fs, const void* X, const int32_t* offset,
                               const int32_t* map1, const void* Wg, const void* Wu, void* A,
                               void* GU, float* part, int E, int h, int f, hipStream_t s) {
  if (fs.grid1 == 0) return hipSuccess;
  GemmParams p{X, offset, map1, Wg, Wu, static_cast<bf16*>(A), nullptr, nullptr, nullptr,
               E, h, f, f, fs.nt1, fs.mt1, part, fs.split_max, fs.grid1};
  p.C2 = static_cast<bf16*>(GU);
  p.gn = fs.gn1;
  launch_gemm<true>(fs.bm1, p, s);
  return hipGetLastError();
}

hipError_t launch_wgrad(const void* A, int lda, const void* B, int ldb, const int32_t* offset,
                        void* C, int E, int M, int N, int64_t rows, int ncu, hipStream_t s) {
  const int units = E * ((M + 255) / 256) * ((N + BN - 1) / BN);
  if (units == 0) return hipSuccess;
  // K: A's row pitch, Nout: B's row pitch (the epilogue writes rows of N)
  GemmParams p{A, offset, nullptr, B, nullptr, static_cast<bf16*>(C), nullptr, nullptr, nullptr,
               E, lda, N, ldb, 0, 0, nullptr, 1, 0};
  p.M = M;
  const int grid = std::min(units, ncu);
  // short tiles gain from the stream (DeepSeek-V3 shape, 128 rows an expert:
  // 20% faster); with long ones the staged epilogue of gemm_wgrad_kernel
  // wins slightly (Mixtral shape, 1024 rows an expert: 2.6%)
  if (rows <= 512 * (int64_t)E && (size_t)M * N * 2 < (size_t)kPastEnd - 256 && N % 8 == 0)
    hipLaunchKernelGGL((gemm_wgrad_stream_kernel<2, 3>), dim3(grid), dim3(64 * kWaves), 0, s, p);
  else
    hipLaunchKernelGGL((gemm_wgrad_kernel<2, 3>), dim3(grid), dim3(64 * kWaves), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_down(const FfnShape& fs, const void* A, const int32_t* offset,
                       const int32_t* map2, const void* Wd, void* Y, float* part, int E, int h,
                       int f, int bf16_, hipStream_t s) {
  if (!bf16_) return hipErrorNotSupported;
  if (fs.grid2 == 0) return hipSuccess;
  GemmParams p{A, offset, map2, Wd, nullptr, static_cast<bf16*>(Y), nullptr, nullptr, nullptr,
               E, f, h, h, fs.nt2, fs.mt2, part, fs.split_max, fs.grid2};
  p.gn = fs.gn2;
  launch_gemm<false>(fs.bm2, p, s, fs.wstream);
  return hipGetLastError();
}

hipError_t launch_dgrad(const FfnShape& fs, const void* A, const int32_t* offset,
                        const int32_t* map2, const void* W0, const void* W1, int K0, void* C,
                        float* part, int E, int N, int K, hipStream_t s) {
  if (fs.grid2 == 0) return hipSuccess;
  GemmParams p{A, offset, map2, W0, W1, static_cast<bf16*>(C), nullptr, nullptr, nullptr,
               E, K, N, N, fs.nt2, fs.mt2, part, fs.split_max, fs.grid2};
  p.K0 = K0;
  p.gn = fs.gn2;  // the product's shape decides, as for the forward down product
  launch_gemm_bt(fs.bm2, p, s);
  return hipGetLastError();
}

hipError_t launch_dgrad_fp8(const FfnShape& fs, const void* A8, const float* sa,
                            const int32_t* offset, const int32_t* map2, const void* W8,
                            const float* sw, void* C, float* part, int E, int N, int K,
                            hipStream_t s) {
  if (fs.grid2 == 0) return hipSuccess;
  GemmParams p{A8, offset, map2, W8, nullptr, static_cast<bf16*>(C), sa, sw, nullptr,
               E, K, N, N, fs.nt2, fs.mt2, part, fs.split_max, fs.grid2};
  launch_gemm_fp8<false>(fs.bm2, p, s);
  return hipGetLastError();
}

hipError_t launch_ffn_f32(const void* X, const int32_t* offset, const void* Wg, const void* Wu,
                          const void* Wd, void* A, void* Y, int64_t rows_max, int E, int h,
                          int f, hipStream_t s) {
  if (rows_max == 0) return hipSuccess;
  const int64_t n1 = rows_max * f, n2 = rows_max * h;
  hipLaunchKernelGGL(gemm_f32_kernel<true>, dim3((unsigned)((n1 + 255) / 256)), dim3(256), 0, s,
                     static_cast<const float*>(X), offset, static_cast<const float*>(Wg),
                     static_cast<const float*>(Wu), static_cast<float*>(A), E, h, f);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(gemm_f32_kernel<false>, dim3((unsigned)((n2 + 255) / 256)), dim3(256), 0, s,
                     static_cast<const float*>(A), offset, static_cast<const float*>(Wd),
                     nullptr, static_cast<float*>(Y), E, f, h);
  return hipGetLastError();
}

}  // namespace moe
