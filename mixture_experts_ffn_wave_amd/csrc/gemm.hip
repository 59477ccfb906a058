// Grouped GEMMs of the MoE layer on gfx950 matrix cores.
//
// One tile engine, two kernel families:
//   row GEMMs   -- output rows are token rows.  Rows come in segments (one per
//                  expert, read from the device offsets array, so the host
//                  never learns the per-expert sizes) or as one dense segment.
//                  Used for gate/up (+SwiGLU epilogue), down, the two dgrad
//                  GEMMs (+SwiGLU-backward epilogue) and the
//                  router's input gradient.
//   wgrad GEMMs -- the contraction runs over a segment's tokens (weight
//                  gradients); both operands are token-major.
//
// Tiles.  A workgroup of 4 waves (2 x 2) computes a BM x BN output tile; each
// wave a (BM/2) x (BN/2) quadrant made of 32x32 MFMA tiles (32x32x16 for
// bf16/f16, eight 32x32x2 steps for f32).  Kernels exist for 128 x 128 and
// (16-bit) 256 x 256 tiles; the plan picks per GEMM.
//
// 16-bit main loop.  Operands go from global memory straight into LDS
// (buffer_load ... lds) through a 4-stage ring of 64-byte k chunks, so loads
// run three chunks ahead of the MFMAs with one barrier per chunk.  Operands
// whose rows are contiguous along K are stored [row][k]; operands that arrive
// k-major (weights read transposed, both operands of the weight gradients)
// are stored [k][row] and turned into MFMA fragments by ds_read_b64_tr_b16.
// Both layouts are XOR-swizzled at 16-byte granularity (no padding, no bank
// conflicts on the fragment reads).  f32 operands are staged through
// registers into padded LDS tiles, double buffered.
//
// MFMA operand roles: the weight-side tile feeds the MFMA "A" operand and the
// token-side tile the "B" operand, so each lane holds output columns of one
// token row.  On the 16-bit path the A rows are read in a permuted order that
// leaves 8 consecutive columns in each run of 8 accumulator registers: every
// epilogue store is 16 bytes.

// Every workgroup works out its own tile from the offsets array (a prefix sum
// over at most 256 segments), and workgroup ids are remapped so that each of
// the 8 XCDs (separate L2 caches; ids are handed out round-robin over them)
// receives a contiguous run of tiles.

#include <mutex>
#include <set>
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "mx_codec.h"

namespace moe {
namespace {

constexpr int NT = 256;          // threads of the register-staged (f32) path: 4 waves
constexpr int KB = 128;          // bytes of k staged per chunk

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16* lds_v4i16_ptr;

// Maps the hardware workgroup id onto a logical tile index in [0, R) so that
// XCD x (= id % 8) gets logical tiles [x*Q, (x+1)*Q).  Returns -1 beyond the work.
__device__ __forceinline__ int xcd_logical(int hw, int R) {
  const int q = (R + 7) >> 3;
  const int y = hw >> 3;
  if (y >= q) return -1;
  const int l = (hw & 7) * q + y;
  return l < R ? l : -1;
}

// Maps the hardware workgroup id onto a logical tile index in [0, R) in
// chunks of C consecutive tiles dealt round-robin over the XCDs: XCD x gets
// chunks x, x + 8, x + 16, ... in that order (the grid is a multiple of 8 C
// workgroups).  For tiles of unequal work (weight gradients of experts with
// skewed token counts) this spreads every expert over all XCDs, where the
// contiguous mapping above would give the busiest experts to one XCD; a chunk
// keeps tiles that share an operand slice together.  Returns -1 beyond the
// work.  (A grid that is a multiple of 8 C also covers xcd_logical.)
__device__ __forceinline__ int xcd_chunked(int hw, int R, int C) {
  const int x = hw & 7, y = hw >> 3;
  const int l = ((y / C) * 8 + x) * C + y % C;
  return l < R ? l : -1;
}

// ------------------------------------------------------------ operand tile --
// ROWS rows of the tile; TR: the source is k-major (rows contiguous along the
// tile's row index, one source row per k).
template <typename T, int ROWS, bool TR>
struct Operand {
  static constexpr int ES = sizeof(T);
  static constexpr int BK = KB / ES;                       // k per chunk
  static constexpr bool HWTR = TR && ES == 2;              // transpose on the read side
  static constexpr int STRIDE = HWTR ? ROWS * ES + 64 : KB + 16;
  static constexpr int BYTES = HWTR ? BK * STRIDE : ROWS * STRIDE;
  // 16-byte chunks each thread moves per K chunk
  static constexpr int NREG = ROWS * KB / 16 / NT;         // = ROWS / 32
  static constexpr int CH = Mma32<T>::kChunks;
  // register-transpose path (f32): 4 k-rows x 16 bytes per thread-block
  static constexpr int VR = 16 / ES;                       // row elements per 16 bytes
  static constexpr int NCG = ROWS / VR;                    // column groups of a k-row
  static constexpr int KG = BK / 4;                        // groups of 4 k-rows
  static_assert(HWTR || !TR || NCG * KG == NT * NREG / 4, "f32 transposed tile geometry");

  u32x4 r[NREG];
  static constexpr bool kRawLds = false;

  // -- loads, normal layout: row pointers are precomputed by the caller --
  // chunk c = tid + NT*s holds row c/8, 16-byte column c%8
  __device__ __forceinline__ static int nrow(int tid, int s) { return (tid + NT * s) >> 3; }
  __device__ __forceinline__ void load_normal(const char* const (&rowp)[NREG], int64_t koff, int tid) {
#pragma unroll
    for (int s = 0; s < NREG; ++s)
      r[s] = rowp[s] ? ld16(rowp[s] + koff + (tid & 7) * 16) : (u32x4){0u, 0u, 0u, 0u};
  }
  __device__ __forceinline__ void stage_normal(char* lds, int tid) const {
#pragma unroll
    for (int s = 0; s < NREG; ++s) {
      const int c = tid + NT * s;
      st16(lds + (c >> 3) * STRIDE + (c & 7) * 16, r[s]);
    }
  }

  // -- loads, k-major source: element (k, row) at base + k*ldk + row*ES, k < kvalid --
  __device__ __forceinline__ void load_kmajor(const char* base, int64_t ldk, int kvalid, int tid) {
    if constexpr (HWTR) {
      constexpr int CPR = ROWS * ES / 16;                  // 16-byte chunks per k-row
#pragma unroll
      for (int s = 0; s < NREG; ++s) {
        const int c = tid + NT * s, k = c / CPR, cc = c % CPR;
        r[s] = (k < kvalid) ? ld16(base + (int64_t)k * ldk + cc * 16) : (u32x4){0u, 0u, 0u, 0u};
      }
    } else {
      // thread-block b covers k-rows 4*kg..4*kg+3 and row elements cg*VR..cg*VR+VR-1
#pragma unroll
      for (int b = 0; b < NREG / 4; ++b) {
        const int blk = tid + NT * b, kg = blk / NCG, cg = blk % NCG;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int k = 4 * kg + i;
          r[4 * b + i] = (k < kvalid) ? ld16(base + (int64_t)k * ldk + cg * 16) : (u32x4){0u, 0u, 0u, 0u};
        }
      }
    }
  }
  __device__ __forceinline__ void stage_kmajor(char* lds, int tid) const {
    if constexpr (HWTR) {
      constexpr int CPR = ROWS * ES / 16;
#pragma unroll
      for (int s = 0; s < NREG; ++s) {
        const int c = tid + NT * s, k = c / CPR, cc = c % CPR;
        st16(lds + k * STRIDE + cc * 16, r[s]);
      }
    } else {
#pragma unroll
      for (int b = 0; b < NREG / 4; ++b) {
        const int blk = tid + NT * b, kg = blk / NCG, cg = blk % NCG;
#pragma unroll
        for (int v = 0; v < VR; ++v) {
          // element v of each of the 4 k-rows -> LDS row cg*VR + v at k offset 4*kg
          u32x4 o = {r[4 * b + 0][v], r[4 * b + 1][v], r[4 * b + 2][v], r[4 * b + 3][v]};
          st16(lds + (cg * VR + v) * STRIDE + (4 * kg) * ES, o);
        }
      }
    }
  }

  // -- MFMA fragment: rows row0 .. row0+31, k16 step ks of the chunk --
  template <bool PERM>
  __device__ __forceinline__ static void frag(u32x4 (&f)[CH], const char* lds, int row0, int ks, int lane) {
    static_assert(!PERM, "the register-staged path keeps the natural row order");
    if constexpr (HWTR) {
      const int g = lane >> 4, i = lane & 15;
      const int k = ks * 16 + 8 * (g >> 1) + (i >> 2);
      const int row = row0 + 16 * (g & 1) + 4 * (i & 3);
      const char* p = lds + k * STRIDE + row * ES;
      const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(p));
      const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(p + 4 * STRIDE));
      const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
      f[0] = (u32x4){ua[0], ua[1], ub[0], ub[1]};
    } else {
      const char* p = lds + (row0 + (lane & 31)) * STRIDE + ks * 16 * ES + (lane >> 5) * 8 * ES;
#pragma unroll
      for (int ch = 0; ch < CH; ++ch) f[ch] = ld16(p + ch * 16);
    }
  }
};

// Row order of the weight-side ("A") fragments on the direct-load path: MFMA
// row i reads tile row perm_row(i) (bits 2 and 3 of i swapped).  The 32x32
// accumulator then holds, in registers 8t .. 8t+7 of lane l, the 8 consecutive
// output columns 16t + 8 (l / 32) + 0..7 of token row l % 32 -- one 16-byte
// store per 8 values instead of two 8-byte ones.
__device__ __forceinline__ int perm_row(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

// Output column (within a 32-column subtile) of accumulator register r of a
// lane in half h = lane / 32.
template <bool PERM>
__device__ __forceinline__ constexpr int acc_col(int r, int h) {
  return PERM ? 16 * (r >> 3) + 8 * h + (r & 7) : 8 * (r >> 2) + 4 * h + (r & 3);
}

// Transposing fragment reads (ds_read_b64_tr_b16) through the builtin: the
// compiler tracks each read and waits only for those an MFMA consumes.  The
// buffer-to-LDS loads are inline assembly (dma4 / dma16 below), so the
// compiler does not see them as LDS writes still in flight and adds no
// vmcnt(0) before these reads; the ring barrier orders them instead.
template <int M>
__device__ __forceinline__ void tr_read(u32x2 (&o)[M], const uint32_t (&a)[M]) {
#pragma unroll
  for (int i = 0; i < M; ++i) {
    const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(uintptr_t)a[i]);
    o[i] = __builtin_bit_cast(u32x2, v);
  }
}

// MFMA work of one chunk for a wave: NS weight-side subtiles (LDS rows
// qrow[ns]) x MS token-side subtiles (LDS rows prow[ms]).  Fragments of
// plain layouts are ordinary LDS loads; those of transposed layouts go
// through tr_read.
template <typename T, typename PO, typename QO, int NS, int MS, int KSTEPS = KB / sizeof(T) / 16,
          bool PERM = false>
__device__ __forceinline__ void mfma_chunk(f32x16 (&acc)[NS][MS], const char* lq, const char* lp,
                                           const int (&qrow)[NS], const int (&prow)[MS], int lane) {
  constexpr int CH = Mma32<T>::kChunks;
  constexpr int NRAW = (QO::kRawLds ? NS : 0) + (PO::kRawLds ? MS : 0);
  if constexpr (NRAW == 0 && PERM) {
    // Every k step's fragments first, then the MFMAs: the k step 0 products
    // start as soon as its fragments arrive while the later ones are read.
    u32x4 fa[KSTEPS][NS][CH], fb[KSTEPS][MS][CH];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) PO::template frag<false>(fb[ks][ms], lp, prow[ms], ks, lane);
#pragma unroll
      for (int ns = 0; ns < NS; ++ns) QO::template frag<PERM>(fa[ks][ns], lq, qrow[ns], ks, lane);
    }
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
      for (int ns = 0; ns < NS; ++ns)
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) Mma32<T>::run(acc[ns][ms], fa[ks][ns], fb[ks][ms]);
    return;
  }
  if constexpr (NRAW > 0 && NRAW * KSTEPS <= 8 && (NRAW * KSTEPS) % 2 == 0) {
    // Every k step's fragments of the chunk at once, plain ones first, then
    // the transposed ones; each MFMA waits only for its own fragments.
    u32x4 fa[KSTEPS][NS][CH], fb[KSTEPS][MS][CH];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      if constexpr (!PO::kRawLds) {
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) PO::template frag<false>(fb[ks][ms], lp, prow[ms], ks, lane);
      }
      if constexpr (!QO::kRawLds) {
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) QO::template frag<PERM>(fa[ks][ns], lq, qrow[ns], ks, lane);
      }
    }
    constexpr int QB = 0, PB = QO::kRawLds ? NS : 0;       // fragment slots of each operand per k step
    uint32_t addr[2 * NRAW * KSTEPS];
    u32x2 raw[2 * NRAW * KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      uint32_t* ak = addr + 2 * NRAW * ks;
      if constexpr (QO::kRawLds) {
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) QO::template frag_addr<PERM>(ak + 2 * (QB + ns), lq, qrow[ns], ks, lane);
      }
      if constexpr (PO::kRawLds) {
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) PO::template frag_addr<false>(ak + 2 * (PB + ms), lp, prow[ms], ks, lane);
      }
    }
    tr_read(raw, addr);
    // every read of the chunk issues before the first MFMA; the MFMAs then
    // run at raised wave priority so a wave that has its fragments keeps the
    // matrix unit while the other waves on the SIMD issue their reads
    __builtin_amdgcn_sched_group_barrier(0x100, 64, 0);    // DS reads
    __builtin_amdgcn_sched_group_barrier(0x008, 64, 0);    // then MFMAs
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const u32x2* rk = raw + 2 * NRAW * ks;
      if constexpr (QO::kRawLds) {
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) {
          const u32x2 lo = rk[2 * (QB + ns)], hi = rk[2 * (QB + ns) + 1];
          fa[ks][ns][0] = (u32x4){lo[0], lo[1], hi[0], hi[1]};
        }
      }
      if constexpr (PO::kRawLds) {
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) {
          const u32x2 lo = rk[2 * (PB + ms)], hi = rk[2 * (PB + ms) + 1];
          fb[ks][ms][0] = (u32x4){lo[0], lo[1], hi[0], hi[1]};
        }
      }
#pragma unroll
      for (int ns = 0; ns < NS; ++ns)
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) Mma32<T>::run(acc[ns][ms], fa[ks][ns], fb[ks][ms]);
    }
    __builtin_amdgcn_s_setprio(0);
    return;
  }
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    u32x4 fa[NS][CH], fb[MS][CH];
    if constexpr (!PO::kRawLds) {
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) PO::template frag<false>(fb[ms], lp, prow[ms], ks, lane);
    }
    if constexpr (!QO::kRawLds) {
#pragma unroll
      for (int ns = 0; ns < NS; ++ns) QO::template frag<PERM>(fa[ns], lq, qrow[ns], ks, lane);
    }
    if constexpr (NRAW > 0) {
      uint32_t addr[2 * NRAW];
      u32x2 raw[2 * NRAW];
      constexpr int QB = 0, PB = QO::kRawLds ? NS : 0;     // fragment slots of each operand
      if constexpr (QO::kRawLds) {
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) QO::template frag_addr<PERM>(addr + 2 * (QB + ns), lq, qrow[ns], ks, lane);
      }
      if constexpr (PO::kRawLds) {
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) PO::template frag_addr<false>(addr + 2 * (PB + ms), lp, prow[ms], ks, lane);
      }
      tr_read(raw, addr);
      if constexpr (QO::kRawLds) {
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) {
          const u32x2 lo = raw[2 * (QB + ns)], hi = raw[2 * (QB + ns) + 1];
          fa[ns][0] = (u32x4){lo[0], lo[1], hi[0], hi[1]};
        }
      }
      if constexpr (PO::kRawLds) {
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) {
          const u32x2 lo = raw[2 * (PB + ms)], hi = raw[2 * (PB + ms) + 1];
          fb[ms][0] = (u32x4){lo[0], lo[1], hi[0], hi[1]};
        }
      }
    }
#pragma unroll
    for (int ns = 0; ns < NS; ++ns)
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) Mma32<T>::run(acc[ns][ms], fa[ns], fb[ms]);
  }
}

// Fragments of one ring chunk, every k step, into registers (the ping-pong
// loop reads them in one phase and multiplies them in the next): weight-side
// rows qrow[ns] (in perm_row order), token-side rows prow[ms].
template <typename PO, typename QO, int NS, int MS, int KSTEPS>
__device__ __forceinline__ void read_chunk_frags(u32x4 (&fa)[KSTEPS][NS], u32x4 (&fb)[KSTEPS][MS], const char* lq,
                                                 const char* lp, const int (&qrow)[NS], const int (&prow)[MS],
                                                 int lane) {
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
      if constexpr (PO::kRawLds) {
        uint32_t ad[2];
        u32x2 raw[2];
        PO::template frag_addr<false>(ad, lp, prow[ms], ks, lane);
        tr_read(raw, ad);
        fb[ks][ms] = (u32x4){raw[0][0], raw[0][1], raw[1][0], raw[1][1]};
      } else {
        u32x4 f[1];
        PO::template frag<false>(f, lp, prow[ms], ks, lane);
        fb[ks][ms] = f[0];
      }
    }
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) {
      if constexpr (QO::kRawLds) {
        uint32_t ad[2];
        u32x2 raw[2];
        QO::template frag_addr<true>(ad, lq, qrow[ns], ks, lane);
        tr_read(raw, ad);
        fa[ks][ns] = (u32x4){raw[0][0], raw[0][1], raw[1][0], raw[1][1]};
      } else {
        u32x4 f[1];
        QO::template frag<true>(f, lq, qrow[ns], ks, lane);
        fa[ks][ns] = f[0];
      }
    }
  }
}

template <typename T, int NS, int MS, int KSTEPS>
__device__ __forceinline__ void mfma_chunk_frags(f32x16 (&acc)[NS][MS], const u32x4 (&fa)[KSTEPS][NS],
                                                 const u32x4 (&fb)[KSTEPS][MS]) {
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
    for (int ns = 0; ns < NS; ++ns)
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) Mma32<T>::run(acc[ns][ms], &fa[ks][ns], &fb[ks][ms]);
}

// ---- MX-fp8 (e4m3 payload, one power-of-two scale per 32 values of k) ----
// v_mfma_scale_f32_32x32x64_f8f6f4 over a 64-k step (two scale blocks): lane
// l supplies operand row l % 32, with payload bytes 0-15 from k 16 h .. +15 of
// the first block and bytes 16-31 from the same offsets of the second block
// (h = l / 32), and the scale byte of block h of that row; the accumulator
// layout is that of the other 32x32 MFMAs.  Which k of a block a byte stands
// for does not change the dot product as long as both operands agree, so only
// the block membership of each byte and each scale matters.
typedef int v8i __attribute__((ext_vector_type(8)));
constexpr int MX_DKB = 128;                 // k bytes (= k values) per ring chunk: 4 scale blocks

// 32 payload bytes of row r: k [64 ks + 16 h, +16) and [64 ks + 32 + 16 h, +16), from a [row][128-byte]
// tile with the 128-byte-row swizzle of DmaRows (chunk c at c ^ ((r >> 1) & 7))
__device__ __forceinline__ v8i mx_frag(const char* lds, int r, int ks, int h) {
  const int c = 4 * ks + h, sw = (r >> 1) & 7;
  const u32x4 lo = ld16(lds + r * MX_DKB + ((c ^ sw) << 4));
  const u32x4 hi = ld16(lds + r * MX_DKB + (((c + 2) ^ sw) << 4));
  return (v8i){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// One 128-k chunk for a wave: weight-side rows qrow[ns] (read in perm_row
// order, as on the 16-bit path), token-side rows prow[ms]; scale tiles are
// [row][4 bytes] (one byte per 32-k block of the chunk).
template <int NS, int MS>
__device__ __forceinline__ void mfma_chunk_mx(f32x16 (&acc)[NS][MS], const char* lq, const char* lp,
                                              const uint8_t* sq, const uint8_t* sp,
                                              const int (&qrow)[NS], const int (&prow)[MS], int lane) {
  constexpr int KS = MX_DKB / 64;
  const int h = lane >> 5;
  if constexpr (NS * MS > 4) {
    // the 256 x 256 tile's waves (8 output subtiles): one k step's fragments
    // at a time, so the chunk's fragments and the 128 accumulators fit the
    // register budget
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      v8i fa[NS], fb[MS];
      int sa[NS], sb[MS];
#pragma unroll
      for (int ns = 0; ns < NS; ++ns) {
        const int r = qrow[ns] + perm_row(lane & 31);
        fa[ns] = mx_frag(lq, r, ks, h);
        sa[ns] = sq[4 * r + 2 * ks + h];
      }
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) {
        const int r = prow[ms] + (lane & 31);
        fb[ms] = mx_frag(lp, r, ks, h);
        sb[ms] = sp[4 * r + 2 * ks + h];
      }
#pragma unroll
      for (int ns = 0; ns < NS; ++ns)
#pragma unroll
        for (int ms = 0; ms < MS; ++ms)
          acc[ns][ms] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[ns], fb[ms], acc[ns][ms], 0, 0, 0, sa[ns],
                                                                          0, sb[ms]);
    }
    return;
  }
  // every k step's fragments and scales first, then the MFMAs
  v8i fa[KS][NS], fb[KS][MS];
  int sa[KS][NS], sb[KS][MS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) {
      const int r = qrow[ns] + perm_row(lane & 31);
      fa[ks][ns] = mx_frag(lq, r, ks, h);
      sa[ks][ns] = sq[4 * r + 2 * ks + h];
    }
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
      const int r = prow[ms] + (lane & 31);
      fb[ks][ms] = mx_frag(lp, r, ks, h);
      sb[ks][ms] = sp[4 * r + 2 * ks + h];
    }
  }
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int ns = 0; ns < NS; ++ns)
#pragma unroll
      for (int ms = 0; ms < MS; ++ms)
        acc[ns][ms] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[ks][ns], fb[ks][ms], acc[ns][ms], 0, 0, 0,
                                                                        sa[ks][ns], 0, sb[ks][ms]);
}

template <int NS, int MS>
__device__ __forceinline__ void zero_acc(f32x16 (&acc)[NS][MS]) {
#pragma unroll
  for (int i = 0; i < NS; ++i)
#pragma unroll
    for (int j = 0; j < MS; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
}


// --------------------------------------------- direct-to-LDS operand tiles --
// 16-bit operands go from global memory straight into LDS with
// buffer_load_dwordx4 ... lds: lane l of an instruction lands 16 bytes at the
// instruction's LDS base + 16 l, and offsets at or past the descriptor's record
// count read as zero (masked rows and tokens cost no branch).  Tiles are
// unpadded and XOR-swizzled at 16-byte granularity so the fragment reads are
// free of bank conflicts:
//   [row][k] tiles (64-byte rows): chunk c of row r sits at c ^ ((r >> 2) & 3)
//   [k][row] tiles: chunk c of k-row k sits at c ^ (4 (k & 3))
// Each wave issues ROWS/64 loads per operand per 64-byte K chunk.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format (gfx9 family)

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}
// The LDS base goes in M0 (set by the compiler from the "{m0}" operand; the
// s_nop covers the M0-write-to-LDS-DMA hazard).  The "memory" clobber keeps
// LDS accesses from moving across; completion is tracked by the explicit
// vmcnt waits of the ring barriers.
__device__ __forceinline__ void dma4(rsrc_t rs, char* lds_lane0, uint32_t voff) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds_lane0;
  asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(rs), "{m0}"(m0) : "memory");
}
__device__ __forceinline__ void dma16(rsrc_t rs, char* lds_lane0, uint32_t voff) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds_lane0;
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rs), "{m0}"(m0) : "memory");
}

// Tile configurations of the direct-load path (BM x BN output tiles):
//   128 x 128: 4 waves (2 x 2), a ring of 64-byte k chunks: 3 stages (48 KB,
//              three workgroups per CU) for the row GEMMs, 4 stages (64 KB,
//              loads three chunks ahead, two workgroups per CU) for the weight
//              gradients, whose workgroups run long K loops;
//   128 x 256: row GEMMs only, 4 waves (2 x 2, 64 x 128 per wave), 3 stages of
//              64-byte chunks (72 KB, two workgroups per CU): a quarter less
//              operand traffic per FLOP than 128 x 128 and twice the MFMAs
//              per wave between barriers;
//   256 x 256: 8 waves (2 along rows x 4 along columns, 128 x 64 per wave), a
//              2-stage ring of 128-byte k chunks (each row's chunk is one full
//              cache line), 128 KB of LDS: one workgroup per CU.
//   256 x 256 ping-pong (PP): 8 waves, waves w and w + 4 on one SIMD, a
//              4-stage ring of 64-byte k chunks (128 KB, one workgroup per
//              CU); group w / 4 computes rows 128 (w / 4) .. (128 x 64 per
//              wave).  Each phase one group multiplies a chunk from fragments
//              already in its registers while the other reads the next
//              chunk's fragments and issues its half of the global loads;
//              a barrier ends every phase, so one wave per SIMD issues
//              MFMAs back to back while its partner waits on memory.
template <int BM, int BN, bool WGRAD, bool PP = false> struct TileCfg;
// WAVES_PER_EU: register budget of the row kernels (3 waves per SIMD for the
// 3-workgroup 128 x 128 tiles: the compiler then keeps the accumulators in
// VGPRs and stays within 168 registers).
template <bool WGRAD> struct TileCfg<128, 128, WGRAD> {
  static constexpr int WM = 2, WN = 2, DKB = 64, NSTG = WGRAD ? 4 : 3, THREADS = 256, WAVES_PER_EU = 3;
};
template <> struct TileCfg<128, 256, false> {
  static constexpr int WM = 2, WN = 2, DKB = 64, NSTG = 3, THREADS = 256, WAVES_PER_EU = 2;
};
template <bool WGRAD> struct TileCfg<256, 256, WGRAD> {
  static constexpr int WM = 2, WN = 4, DKB = 128, NSTG = 2, THREADS = 512, WAVES_PER_EU = 2;
};
template <bool WGRAD> struct TileCfg<256, 256, WGRAD, true> {
  static constexpr int WM = 2, WN = 4, DKB = 64, NSTG = 4, THREADS = 512, WAVES_PER_EU = 2;
};

// vmcnt(n) with the other counters left alone (gfx9 s_waitcnt encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

template <int ROWS, int NW, int DKB>
struct DmaRows {                                   // [row][k], DKB bytes per row; NW waves load
  static constexpr int CPRW = DKB / 16;            // 16-byte chunks per row
  static constexpr int RPI = 1024 / DKB;           // rows per load instruction
  static constexpr int BYTES = ROWS * DKB;
  static constexpr int NI = BYTES / 1024 / NW;     // load instructions per wave per chunk
  static_assert(NI >= 1 && NI * 1024 * NW == BYTES, "tile rows must split evenly over the waves");
  static_assert(DKB == 64 || DKB == 128, "chunk width");
  static constexpr bool kRawLds = false;
  // 64-byte rows: 4 rows fill the 256-byte bank space, rows r and r+4 differ
  // by the swizzle; 128-byte rows: 2 rows fill it, rows 2j and 2j+1 get
  // swizzle j (mod 8).  Either way 16 consecutive (or bit-2/3-swapped) rows
  // read at one chunk index hit 16 different 16-byte bank groups.
  __device__ __forceinline__ static int swz(int r) { return DKB == 64 ? (r >> 2) & 3 : (r >> 1) & 7; }
  __device__ __forceinline__ static int row_of(int w, int s, int lane) { return RPI * (w + NW * s) + lane / CPRW; }
  __device__ __forceinline__ static int gchunk(int row, int lane) { return (lane % CPRW) ^ swz(row); }
  __device__ __forceinline__ static int lds_off(int w, int s) { return RPI * (w + NW * s) * DKB; }
  template <bool PERM>
  __device__ __forceinline__ static void frag(u32x4 (&f)[1], const char* lds, int row0, int ks, int lane) {
    const int r = row0 + (PERM ? perm_row(lane & 31) : (lane & 31));
    const int c = ks * 2 + (lane >> 5);
    f[0] = ld16(lds + r * DKB + ((c ^ swz(r)) << 4));
  }
};

template <int ROWS, int NW, int DKB>
struct DmaKmajor {                                 // [k][row], DKB/2 k-rows per chunk; NW waves load
  static constexpr int KROWS = DKB / 2;
  static constexpr int RB = ROWS * 2;              // bytes per k-row
  static constexpr int CPR = RB / 16;              // 16-byte chunks per k-row
  static constexpr int KPI = 1024 / RB;            // k-rows per load instruction
  static constexpr int BYTES = KROWS * RB;
  static constexpr int NI = BYTES / 1024 / NW;
  static_assert(NI >= 1 && NI * 1024 * NW == BYTES, "tile must split evenly over the waves");
  static_assert(CPR >= 16, "swizzle needs at least 16 chunks per k-row");
  // Fragments of this layout are read with ds_read_b64_tr_b16 (tr_read).
  static constexpr bool kRawLds = true;
  __device__ __forceinline__ static int k_of(int w, int s, int lane) { return KPI * (w + NW * s) + lane / CPR; }
  __device__ __forceinline__ static int gchunk(int k, int lane) { return (lane % CPR) ^ (4 * (k & 3)); }
  __device__ __forceinline__ static int lds_off(int w, int s) { return KPI * (w + NW * s) * RB; }
  // LDS addresses of the two transposing reads (k and k + 4) that form the
  // fragment of rows row0 .. row0+31, k16 step ks
  template <bool PERM>
  __device__ __forceinline__ static void frag_addr(uint32_t* a, const char* lds, int row0, int ks, int lane) {
    const int g = lane >> 4, i = lane & 15;
    const int k = ks * 16 + 8 * (g >> 1) + (i >> 2);
    // this lane addresses the 4-row block that MFMA rows 16 (g & 1) + 4 (i & 3) + 0..3 receive
    const int rb = 16 * (g & 1) + 4 * (i & 3);
    const int row = row0 + (PERM ? perm_row(rb) : rb);
    const char* p = lds + k * RB + (((row >> 3) ^ (4 * (k & 3))) << 4) + (row & 7) * 2;
    a[0] = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
    a[1] = a[0] + 4 * RB;
  }
};

// Barrier before chunk kc of the ring.  This wave's loads of chunk kc have
// landed once at most the (up to NSTG-2) later chunks' loads are outstanding;
// its LDS reads of chunk kc-1 have returned (lgkmcnt(0)); s_barrier then makes
// both true for the whole workgroup.  __syncthreads() would add a release
// fence that waits for every outstanding load, draining the ring.  The empty
// asm statements keep the compiler from moving memory accesses across.
template <int LPC, int NSTG>
__device__ __forceinline__ void ring_barrier(int remaining) {
  const int ahead = remaining < NSTG - 2 ? remaining : NSTG - 2;   // chunks issued after this one
  asm volatile("" ::: "memory");
  if (ahead >= 2) wait_vmcnt<2 * LPC>();
  else if (ahead == 1) wait_vmcnt<LPC>();
  else wait_vmcnt<0>();
  __builtin_amdgcn_s_waitcnt(0xC07F);                 // lgkmcnt(0), vmcnt/expcnt untouched
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Barrier before the last chunk when PENDING later loads (issued after that
// chunk's, e.g. the epilogue's first G/U rows) may stay in flight.
template <int PENDING>
__device__ __forceinline__ void ring_barrier_last() {
  asm volatile("" ::: "memory");
  wait_vmcnt<PENDING>();
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// --------------------------------------------------------------- row GEMM ---
// MX: operands are MX-fp8 payload bytes (T = uint8_t) with scale bytes in
// a.Ps / a.Qs, both operands K-contiguous rows (transposes are done by the
// quantiser), outputs bf16.
// LO (SwiGLU backward, 16-bit): also write the rounding remainders of
// [dG | dU] and of the w H rows to a.C_lo / a.C2_lo.
template <typename T, int BM, int BN, int OP, int EPI, int WM, int WN, bool MX = false, bool PP = false,
          bool LO = false>
__device__ __forceinline__ void row_gemm_body(const RowGemmArgs& a, char* smem) {
  constexpr int ES = sizeof(T);
  using TO = std::conditional_t<MX, __bf16, T>;               // output / saved-activation type
  // saved [G | U]: f32 for a bf16 layer (kernels.h, gu_dtype), else TO
  constexpr bool GUF32 = !MX && std::is_same_v<T, __bf16>;
  using TG = std::conditional_t<GUF32, float, TO>;
  constexpr int NW = WM * WN;                                  // waves: WM along rows, WN along columns
  static_assert(ES == 2 || MX || NW == 4, "the register-staged path runs 4 waves");
  static_assert(!MX || (ES == 1 && ((BM == 128 && BN == 128 && NW == 4) || (BM == 256 && BN == 256 && NW == 8))),
                "MX row tiles: 128 x 128 with 4 waves or 256 x 256 with 8");
  constexpr bool QT = !MX && (OP == OP_DOWN_DGRAD || OP == OP_GU_DGRAD || OP == OP_ROUTER_DX);
  using TOP = std::conditional_t<MX, __bf16, T>;              // (register-path operand type; unused for MX)
  using PO = Operand<TOP, BM, false>;
  using QO = Operand<TOP, BN, QT>;
  constexpr int BK = MX ? MX_DKB : PO::BK;
  constexpr int TILE_N = (OP == OP_GU_FWD) ? BN / 2 : BN;    // output (H) columns per tile
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MS = WTM / 32, NS = WTN / 32;
  constexpr int STAGE = PO::BYTES + QO::BYTES;

  static_assert(!PP || (ES == 2 && BM == 256 && BN == 256 && WM == 2 && WN == 4), "ping-pong tile");
  constexpr int DKB = MX ? MX_DKB : TileCfg<BM, BN, false, PP>::DKB;
  constexpr int NSTG = MX ? 2 : TileCfg<BM, BN, false, PP>::NSTG;
  constexpr int SC_OFF = NSTG * (BM + BN) * DKB;                // MX scale tiles follow the payload ring
  constexpr int SCAN_OFF = MX ? SC_OFF + NSTG * (BM + BN) * 4 : ((ES == 2) ? NSTG * (BM + BN) * DKB : 2 * STAGE);
  int* s_scan = reinterpret_cast<int*>(smem + SCAN_OFF);      // [NW] wave sums, [NW..NW+1] located tile
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int n_ntiles = a.N / TILE_N;

  // ---- which (segment, m-tile, n-tile) this workgroup computes
  int my_nt = 0;
  if (tid < a.G) {
    const int64_t len = a.offsets ? (int64_t)(a.offsets[tid + 1] - a.offsets[tid]) : a.M;
    my_nt = (int)((len + BM - 1) / BM);
  }
  int incl = my_nt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) s_scan[wave] = incl;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int sw = s_scan[w];
    before += (w < wave) ? sw : 0;
    total += sw;
  }
  const int start = before + incl - my_nt;
  const int logical = xcd_logical(blockIdx.x, total * n_ntiles);
  if (logical < 0) return;                                    // uniform across the workgroup
  const int mt = logical / n_ntiles, ntile = logical - mt * n_ntiles;
  if (tid < a.G && mt >= start && mt < start + my_nt) { s_scan[NW] = tid; s_scan[NW + 1] = mt - start; }
  __syncthreads();
  const int g = s_scan[NW];
  const int64_t seg0 = a.offsets ? a.offsets[g] : 0;
  const int64_t seg1 = a.offsets ? a.offsets[g + 1] : a.M;
  const int64_t row0 = seg0 + (int64_t)s_scan[NW + 1] * BM;
  const int rows = (int)((seg1 - row0) < BM ? (seg1 - row0) : BM);
  const int n0 = ntile * TILE_N;

  const char* Pb = static_cast<const char*>(a.P);
  const char* Qb = static_cast<const char*>(a.Q) + (int64_t)g * a.q_group_stride * ES;
  // ping-pong: group wave / 4 owns a row half, its four waves (one per SIMD) the column quarters
  const int wm = PP ? wave / WN : wave % WM, wn = PP ? wave % WN : wave / WM;
  int qrow[NS], prow[MS];
#pragma unroll
  for (int ns = 0; ns < NS; ++ns) {
    // gate/up: the wave's first NS/2 subtiles are gate rows, the rest the matching up rows
    if constexpr (OP == OP_GU_FWD)
      qrow[ns] = (ns < NS / 2) ? wn * (WTN / 2) + ns * 32 : BN / 2 + wn * (WTN / 2) + (ns - NS / 2) * 32;
    else
      qrow[ns] = wn * WTN + ns * 32;
  }
#pragma unroll
  for (int ms = 0; ms < MS; ++ms) prow[ms] = wm * WTM + ms * 32;
  f32x16 acc[NS][MS];
  zero_acc(acc);
  const int nk = a.K / BK;

  // Accumulator register layout: runs of RUN consecutive output columns, run t
  // starting at column RSTEP*t + RUN*(lane/32) of a 32-column subtile.
  constexpr bool PERM = (ES == 2) || MX;
  constexpr int RUN = PERM ? 8 : 4, NRUN = 16 / RUN, RSTEP = PERM ? 16 : 8;
  static_assert(acc_col<PERM>(RUN, 0) == RSTEP && acc_col<PERM>(0, 1) == RUN, "run layout");
  const int h = lane >> 5;

  // ---- epilogue staging geometry (16-bit path).  The epilogue runs in MS
  // passes of SR = 32 WM rows (row subtile ms of every wave row); each pass
  // goes through LDS so that global loads and stores move whole rows of the
  // tile: row r of a staged array is RB bytes, 16-byte chunk c at position
  // c ^ (r & 7) (conflict-free both for the MFMA-layout accesses, 8 rows per
  // chunk index, and for the row-wise ones).
  constexpr int SR = 32 * WM;
  constexpr int RB = EPI == EPI_STORE_F32 ? BN * 4 : (EPI == EPI_SWIGLU_FWD ? BN : BN * 2);
  // SwiGLU backward: the w H rows (C2) go through a third staged array where
  // it fits in the ring's LDS, else straight from registers
  // (bf16 and f32 layers; an f16 layer's down weight gradient reads w dy and H)
  constexpr bool WH = EPI == EPI_SWIGLU_BWD && !MX && !std::is_same_v<T, _Float16>;
  constexpr bool WH_STAGED = WH && 3 * 32 * WM * RB <= NSTG * (BM + BN) * DKB;
  constexpr int NARR = (EPI == EPI_SWIGLU_FWD || WH_STAGED) ? 3 : (EPI == EPI_SWIGLU_BWD ? 2 : 1);
  constexpr int CPR = RB / 16;                              // chunks per staged row
  constexpr int SITER = SR * CPR / (64 * NW);               // row-wise chunks per thread per array
  static_assert(!PERM || (CPR >= 8 && SITER >= 1 && SITER * 64 * NW == SR * CPR), "staging geometry");
  // tile row of staged row sr in pass ms
  auto srow = [&](int sr, int ms) { return (sr / 32) * WTM + ms * 32 + (sr % 32); };
  static_assert(!PERM || NARR * SR * RB <= NSTG * (BM + BN) * DKB, "staging fits in the ring's LDS");
  // first packed [G | U] column of this tile's H columns n0.. (SwiGLU epilogues)
  const int gblk = n0 / a.sub;
  const int gcol0 = gblk * 2 * a.sub + (n0 - gblk * a.sub);

  // SwiGLU backward: the saved G and U of one pass, whole rows of the tile.
  // Buffer loads bounded by the tile's rows (rows past them read as zero), so
  // every lane issues exactly 2 SITER loads, which the vmcnt accounting of
  // the prefetch below relies on.
  auto load_gu_rows = [&](u32x4 (&dst)[2][PERM ? SITER : 1], int ms) {
    const rsrc_t grs = make_rsrc(static_cast<const TO*>(a.aux) + row0 * a.ldaux, (uint32_t)(rows * a.ldaux * sizeof(TO)));
#pragma unroll
    for (int i = 0; i < SITER; ++i) {
      const int q = tid + 64 * NW * i, sr = q / CPR, c = q % CPR;
      const uint32_t off = (uint32_t)((srow(sr, ms) * a.ldaux + gcol0 + c * 8) * sizeof(TO));
      dst[0][i] = __builtin_amdgcn_raw_buffer_load_b128(grs, off, 0, 0);
      dst[1][i] = __builtin_amdgcn_raw_buffer_load_b128(grs, off + (uint32_t)(a.sub * sizeof(TO)), 0, 0);
    }
  };
  // The first pass's G/U rows are loaded during the last two k chunks, where
  // their latency hides behind MFMAs (128 x 128 tiles: 32 more VGPRs there,
  // still three workgroups per CU); each later pass's rows are loaded while
  // the previous pass computes.
  constexpr bool GU_PRE = PERM && !GUF32 && EPI == EPI_SWIGLU_BWD && BM == 128 && BN == 128;
  // Ping-pong tiles (one workgroup per CU, nothing else to hide a pass's
  // G/U load behind): the first pass's rows are loaded during the last two
  // chunks of the main loop and each later pass's rows while the previous
  // pass computes and stores (32 more VGPRs, within the 256 that two waves
  // per SIMD allow).
  constexpr bool GU_PIPE = PERM && !GUF32 && EPI == EPI_SWIGLU_BWD && PP;
  u32x4 gun[2][PERM ? SITER : 1];                           // (unused unless GU_PRE or GU_PIPE)
  bool gu_first = false;                                    // GU_PIPE: the first pass's rows are in gun
  // The last two chunks of a ring main loop, with the first pass's G/U loads
  // issued after every chunk's loads (so a vmcnt of 2 SITER before the last
  // chunk still means that chunk has landed).
  auto gu_prefetch_tail = [&](int nkd, auto barrier, auto issue_ahead, auto compute) {
    if (nkd >= 2) {
      barrier(1);
      issue_ahead(nkd - 2);
      asm volatile("" ::: "memory");                          // G/U loads after the chunk loads
      load_gu_rows(gun, 0);
      compute(nkd - 2);
    } else {
      load_gu_rows(gun, 0);
    }
    if (nkd >= 1) {
      ring_barrier_last<2 * SITER>();
      compute(nkd - 1);
    }
  };

  if constexpr (MX) {
    // ---------------- direct-to-LDS main loop, MX-fp8 payload + scale tiles
    using PD = DmaRows<BM, NW, MX_DKB>;
    using QD = DmaRows<BN, NW, MX_DKB>;
    constexpr int DSTAGE = PD::BYTES + QD::BYTES;
    constexpr int SSTAGE = (BM + BN) * 4;
    const int64_t pls = a.ldp / 32, qls = a.ldq / 32;          // scale bytes per row
    // token rows: this tile's rows of P, or rows of P picked by a.gather (then
    // the descriptor spans all of P and rows past the tile read past its end)
    const bool gat = a.gather != nullptr;
    const rsrc_t prs = gat ? make_rsrc(Pb, (uint32_t)(a.p_rows * a.ldp))
                           : make_rsrc(Pb + row0 * a.ldp, (uint32_t)(rows * a.ldp));
    auto prow_src = [&](int r) -> int64_t {
      return gat ? (r < rows ? (int64_t)a.gather[row0 + r] : a.p_rows) : (int64_t)r;
    };
    uint32_t poff[PD::NI];
#pragma unroll
    for (int s2 = 0; s2 < PD::NI; ++s2) {
      const int r = PD::row_of(wave, s2, lane);
      poff[s2] = (uint32_t)(prow_src(r) * a.ldp + PD::gchunk(r, lane) * 16);
    }
    // weight-side row of tile row q
    auto qsrc_row = [&](int q) -> int64_t {
      if constexpr (OP == OP_GU_FWD) {
        const int blk = n0 / a.sub, r0 = n0 - blk * a.sub;
        return blk * 2 * a.sub + (q < BN / 2 ? r0 + q : a.sub + r0 + (q - BN / 2));
      } else {
        return n0 + q;
      }
    };
    uint32_t qoff[QD::NI];
#pragma unroll
    for (int s2 = 0; s2 < QD::NI; ++s2) {
      const int q = QD::row_of(wave, s2, lane);
      qoff[s2] = (uint32_t)(qsrc_row(q) * a.ldq + QD::gchunk(q, lane) * 16);
    }
    // scale rows: wave 0/1 load P rows 0-63 / 64-127, wave 2/3 Q rows 0-63 / 64-127
    // scale rows: the first BM / 64 waves load P's rows 64 w .. 64 w + 63, the
    // others Q's
    static_assert(64 * NW == BM + BN, "one wave per 64 scale rows");
    const bool sq_side = wave >= BM / 64;
    const int swave = sq_side ? wave - BM / 64 : wave;
    const int srow_t = swave * 64 + lane;
    const uint8_t* qsb = a.Qs + (int64_t)g * (a.q_group_stride / 32);
    const rsrc_t psrs = gat ? make_rsrc(a.Ps, (uint32_t)(a.p_rows * pls))
                            : make_rsrc(a.Ps + row0 * pls, (uint32_t)(rows * pls));
    const uint32_t soff = sq_side ? (uint32_t)(qsrc_row(srow_t) * qls) : (uint32_t)(prow_src(srow_t) * pls);
    auto issue = [&](int kc, int st) {
      char* stage = smem + st * DSTAGE;
#pragma unroll
      for (int s2 = 0; s2 < PD::NI; ++s2) dma16(prs, stage + PD::lds_off(wave, s2), poff[s2] + (uint32_t)kc);
      const rsrc_t qrs = make_rsrc(Qb + kc, 0x7fffffffu);
#pragma unroll
      for (int s2 = 0; s2 < QD::NI; ++s2) dma16(qrs, stage + PD::BYTES + QD::lds_off(wave, s2), qoff[s2]);
      char* sst = smem + SC_OFF + st * SSTAGE + (sq_side ? BM * 4 : 0) + swave * 64 * 4;
      if (sq_side) dma4(make_rsrc(qsb + kc / 32, 0x7fffffffu), sst, soff);
      else dma4(psrs, sst, soff + (uint32_t)(kc / 32));
    };
    constexpr int LPC = PD::NI + QD::NI + 1;
    const int nkd = a.K / MX_DKB;
#pragma unroll
    for (int c = 0; c < NSTG - 1; ++c)
      if (c < nkd) issue(c * MX_DKB, c);
    auto issue_ahead = [&](int kc) {
      if (kc + NSTG - 1 < nkd) issue((kc + NSTG - 1) * MX_DKB, (kc + NSTG - 1) % NSTG);
    };
    auto compute = [&](int kc) {
      const int st = kc % NSTG;
      const char* buf = smem + st * DSTAGE;
      const uint8_t* sbuf = reinterpret_cast<const uint8_t*>(smem + SC_OFF + st * SSTAGE);
      mfma_chunk_mx<NS, MS>(acc, buf + PD::BYTES, buf, sbuf + BM * 4, sbuf, qrow, prow, lane);
    };
    const int nloop = GU_PRE ? nkd - 2 : nkd;
    for (int kc = 0; kc < nloop; ++kc) {
      ring_barrier<LPC, NSTG>(nkd - 1 - kc);
      issue_ahead(kc);
      compute(kc);
    }
    if constexpr (GU_PRE) gu_prefetch_tail(nkd, ring_barrier<LPC, NSTG>, issue_ahead, compute);
  } else if constexpr (ES == 2 && PP) {
    // ---------------- ping-pong main loop (16-bit, 256 x 256, 8 waves)
    // Group 0 (waves 0-3) streams the token-side tile, group 1 (waves 4-7) the
    // weight-side tile, each half of a chunk issued by four waves.  Every wave
    // runs the same straight line per chunk c: a memory phase (read chunk c's
    // fragments into registers, issue its half of chunk c + NSTG - 1 into the
    // slot of chunk c - 1, wait for its own loads of chunk c + 1) and a
    // compute phase (the chunk's MFMAs from registers), a barrier after each.
    // Group 1 starts one barrier late and group 0 ends with one more, so the
    // two groups are a phase apart: while one wave of a SIMD issues MFMAs, its
    // partner waits on memory.  (s_barrier pairs the k-th arrival of every
    // wave, wherever in the program it is.)  Chunk c is read by group 0 in the
    // phase after barrier 2c + 1 and by group 1 after barrier 2c + 2; each
    // wave's memory phase for chunk c - 1 ends before barrier 2c + 1 with its
    // own loads of chunk c landed, so that barrier makes chunk c readable, and
    // the slot of chunk c - 1 is rewritten only after both groups' reads of
    // it have returned (lgkmcnt(0) before their barriers).
    constexpr int NWL = 4;                           // waves loading each half
    using PD = DmaRows<BM, NWL, DKB>;
    using QD = std::conditional_t<QT, DmaKmajor<BN, NWL, DKB>, DmaRows<BN, NWL, DKB>>;
    static_assert(PD::NI == QD::NI, "both halves issue the same number of loads per wave");
    constexpr int DSTAGE = PD::BYTES + QD::BYTES;
    constexpr int DBKE = DKB / ES;                    // k elements per chunk
    constexpr int KSTEPS = DKB / 32;
    constexpr int LPH = PD::NI;                       // loads per wave per chunk half
    const int grp = wave >> 2, wq = wave & 3;
    const bool gat = a.gather != nullptr;
    const rsrc_t prs = gat ? make_rsrc(Pb, (uint32_t)(a.p_rows * a.ldp * ES))
                           : make_rsrc(Pb + row0 * a.ldp * ES, (uint32_t)(rows * a.ldp * ES));
    uint32_t off[LPH];
    const char* qbase = Qb;
    int64_t qldk = 0;
    if (grp == 0) {
#pragma unroll
      for (int s2 = 0; s2 < LPH; ++s2) {
        const int r = PD::row_of(wq, s2, lane);
        const int64_t src = gat ? (r < rows ? (int64_t)a.gather[row0 + r] : a.p_rows) : (int64_t)r;
        off[s2] = (uint32_t)(src * a.ldp * ES + PD::gchunk(r, lane) * 16);
      }
    } else {
      if constexpr (!QT) {
#pragma unroll
        for (int s2 = 0; s2 < LPH; ++s2) {
          const int q = QD::row_of(wq, s2, lane);
          int64_t roff;
          if constexpr (OP == OP_GU_FWD) {
            const int blk = n0 / a.sub, r0 = n0 - blk * a.sub;
            const int wrow = blk * 2 * a.sub + (q < BN / 2 ? r0 + q : a.sub + r0 + (q - BN / 2));
            roff = (int64_t)wrow * a.ldq;
          } else {
            roff = (int64_t)(n0 + q) * a.sub;         // OP_DOWN_FWD, block part added per chunk
          }
          off[s2] = (uint32_t)(roff * ES + QD::gchunk(q, lane) * 16);
        }
      } else {
        if constexpr (OP == OP_DOWN_DGRAD) {
          const int blk = n0 / a.sub, c0 = n0 - blk * a.sub;
          qbase = Qb + ((int64_t)blk * a.K * a.sub + c0) * ES;
          qldk = (int64_t)a.sub * ES;
        } else {
          qbase = Qb + (int64_t)n0 * ES;
          qldk = a.ldq * ES;
        }
#pragma unroll
        for (int s2 = 0; s2 < LPH; ++s2) {
          const int k = QD::k_of(wq, s2, lane);
          off[s2] = (uint32_t)(k * qldk + QD::gchunk(k, lane) * 16);
        }
      }
    }
    // this wave's half of chunk c (group 0: token rows, group 1: weight rows)
    auto issue_half = [&](int c) {
      char* stage = smem + (c % NSTG) * DSTAGE;
      const int kc = c * DBKE;
      if (grp == 0) {
#pragma unroll
        for (int s2 = 0; s2 < LPH; ++s2) dma16(prs, stage + PD::lds_off(wq, s2), off[s2] + (uint32_t)(kc * ES));
      } else if constexpr (!QT) {
        int64_t koff = (int64_t)kc * ES;
        if constexpr (OP == OP_DOWN_FWD) {
          const int blk = kc / a.sub, kk = kc - blk * a.sub;
          koff = ((int64_t)blk * a.N * a.sub + kk) * ES;
        }
        const rsrc_t qrs = make_rsrc(qbase + koff, 0x7fffffffu);
#pragma unroll
        for (int s2 = 0; s2 < LPH; ++s2) dma16(qrs, stage + PD::BYTES + QD::lds_off(wq, s2), off[s2]);
      } else {
        const rsrc_t qrs = make_rsrc(qbase + (int64_t)kc * qldk, (uint32_t)(QD::KROWS * qldk));
#pragma unroll
        for (int s2 = 0; s2 < LPH; ++s2) dma16(qrs, stage + PD::BYTES + QD::lds_off(wq, s2), off[s2]);
      }
    };
    // wait until this wave's loads of chunk c have landed (later chunks of its half may be in flight)
    auto wait_chunk = [&](int c, int nkd) {
      const int later = (nkd - 1 - c) < NSTG - 2 ? (nkd - 1 - c) : NSTG - 2;
      asm volatile("" ::: "memory");
      if (later >= 2) wait_vmcnt<2 * LPH>();
      else if (later == 1) wait_vmcnt<LPH>();
      else wait_vmcnt<0>();
    };
    auto phase_barrier = [&]() {
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };
    static_assert(NSTG - 2 <= 2, "wait_chunk covers at most two later chunks");
    const int nkd = a.K / DBKE;
#pragma unroll
    for (int c = 0; c < NSTG - 1; ++c)
      if (c < nkd) issue_half(c);
    if (nkd > 0) wait_chunk(0, nkd);
    phase_barrier();
    if (grp == 1) phase_barrier();                  // one phase behind group 0
    u32x4 fa[KSTEPS][NS], fb[KSTEPS][MS];
    // SwiGLU backward: the first epilogue pass's G/U rows are loaded in the
    // last-but-one chunk, after the ring's last loads, so the wait for the
    // last chunk allows those 2 SITER loads to stay in flight
    const int gu_at = nkd >= 2 ? nkd - 2 : 0;
    for (int c = 0; c < nkd; ++c) {
      const char* buf = smem + (c % NSTG) * DSTAGE;
      read_chunk_frags<PD, QD, NS, MS, KSTEPS>(fa, fb, buf + PD::BYTES, buf, qrow, prow, lane);
      if (c + NSTG - 1 < nkd) issue_half(c + NSTG - 1);
      if constexpr (GU_PIPE) {
        if (c == gu_at) {
          asm volatile("" ::: "memory");
          load_gu_rows(gun, 0);
          gu_first = true;
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);           // lgkmcnt(0): fragments in registers, slot read
      if (c + 1 < nkd) {
        if (GU_PIPE && c == gu_at) {
          asm volatile("" ::: "memory");
          wait_vmcnt<2 * SITER>();                   // chunk c + 1 = the last; only G/U after it
        } else {
          wait_chunk(c + 1, nkd);
        }
      }
      phase_barrier();
      __builtin_amdgcn_s_setprio(1);
      mfma_chunk_frags<T, NS, MS, KSTEPS>(acc, fa, fb);
      __builtin_amdgcn_s_setprio(0);
      phase_barrier();
    }
    if (grp == 0) phase_barrier();                  // as many barriers as group 1
  } else if constexpr (ES == 2) {
    // ---------------- direct-to-LDS main loop (16-bit types)
    using PD = DmaRows<BM, NW, DKB>;
    using QD = std::conditional_t<QT, DmaKmajor<BN, NW, DKB>, DmaRows<BN, NW, DKB>>;
    constexpr int DSTAGE = PD::BYTES + QD::BYTES;
    constexpr int DBKE = DKB / ES;                    // k elements per chunk
    // token rows of this tile: rows >= `rows` fall outside the descriptor and
    // read as zero; gathered rows (a.gather) are addressed in all of P, rows
    // past the tile pointing one row past its end
    const bool gat = a.gather != nullptr;
    const rsrc_t prs = gat ? make_rsrc(Pb, (uint32_t)(a.p_rows * a.ldp * ES))
                           : make_rsrc(Pb + row0 * a.ldp * ES, (uint32_t)(rows * a.ldp * ES));
    uint32_t poff[PD::NI];
#pragma unroll
    for (int s2 = 0; s2 < PD::NI; ++s2) {
      const int r = PD::row_of(wave, s2, lane);
      const int64_t src = gat ? (r < rows ? (int64_t)a.gather[row0 + r] : a.p_rows) : (int64_t)r;
      poff[s2] = (uint32_t)(src * a.ldp * ES + PD::gchunk(r, lane) * 16);
    }
    uint32_t qoff[QD::NI];
    const char* qbase;
    int64_t qldk = 0;
    if constexpr (!QT) {
      qbase = Qb;
#pragma unroll
      for (int s2 = 0; s2 < QD::NI; ++s2) {
        const int q = QD::row_of(wave, s2, lane);
        int64_t roff;
        if constexpr (OP == OP_GU_FWD) {
          const int blk = n0 / a.sub, r0 = n0 - blk * a.sub;
          const int wrow = blk * 2 * a.sub + (q < BN / 2 ? r0 + q : a.sub + r0 + (q - BN / 2));
          roff = (int64_t)wrow * a.ldq;
        } else {
          roff = (int64_t)(n0 + q) * a.sub;         // OP_DOWN_FWD, block part added per chunk
        }
        qoff[s2] = (uint32_t)(roff * ES + QD::gchunk(q, lane) * 16);
      }
    } else {
      if constexpr (OP == OP_DOWN_DGRAD) {
        const int blk = n0 / a.sub, c0 = n0 - blk * a.sub;
        qbase = Qb + ((int64_t)blk * a.K * a.sub + c0) * ES;
        qldk = (int64_t)a.sub * ES;
      } else {
        qbase = Qb + (int64_t)n0 * ES;
        qldk = a.ldq * ES;
      }
#pragma unroll
      for (int s2 = 0; s2 < QD::NI; ++s2) {
        const int k = QD::k_of(wave, s2, lane);
        qoff[s2] = (uint32_t)(k * qldk + QD::gchunk(k, lane) * 16);
      }
    }
    auto issue = [&](int kc, char* stage) {
#pragma unroll
      for (int s2 = 0; s2 < PD::NI; ++s2) dma16(prs, stage + PD::lds_off(wave, s2), poff[s2] + (uint32_t)(kc * ES));
      if constexpr (!QT) {
        int64_t koff = (int64_t)kc * ES;
        if constexpr (OP == OP_DOWN_FWD) {
          const int blk = kc / a.sub, kk = kc - blk * a.sub;
          koff = ((int64_t)blk * a.N * a.sub + kk) * ES;
        }
        const rsrc_t qrs = make_rsrc(qbase + koff, 0x7fffffffu);
#pragma unroll
        for (int s2 = 0; s2 < QD::NI; ++s2) dma16(qrs, stage + PD::BYTES + QD::lds_off(wave, s2), qoff[s2]);
      } else {
        const rsrc_t qrs = make_rsrc(qbase + (int64_t)kc * qldk, (uint32_t)(QD::KROWS * qldk));
#pragma unroll
        for (int s2 = 0; s2 < QD::NI; ++s2) dma16(qrs, stage + PD::BYTES + QD::lds_off(wave, s2), qoff[s2]);
      }
    };
    constexpr int LPC = PD::NI + QD::NI;             // loads per wave per chunk
    const int nkd = a.K / DBKE;
#pragma unroll
    for (int c = 0; c < NSTG - 1; ++c)
      if (c < nkd) issue(c * DBKE, smem + c * DSTAGE);
    auto issue_ahead = [&](int kc) {
      if (kc + NSTG - 1 < nkd) issue((kc + NSTG - 1) * DBKE, smem + ((kc + NSTG - 1) % NSTG) * DSTAGE);
    };
    auto compute = [&](int kc) {
      const char* buf = smem + (kc % NSTG) * DSTAGE;
      mfma_chunk<T, PD, QD, NS, MS, DKB / 32, true>(acc, buf + PD::BYTES, buf, qrow, prow, lane);
    };
    const int nloop = GU_PRE ? nkd - 2 : nkd;
    for (int kc = 0; kc < nloop; ++kc) {
      ring_barrier<LPC, NSTG>(nkd - 1 - kc);          // chunk kc landed everywhere; kc-1 consumed
      issue_ahead(kc);
      compute(kc);
    }
    if constexpr (GU_PRE) gu_prefetch_tail(nkd, ring_barrier<LPC, NSTG>, issue_ahead, compute);
  } else {
  // ---------------- register-staged main loop (f32)
  // ---- row pointers (normal operands) / k-major base (transposed weight)
  const char* prowp[PO::NREG];
#pragma unroll
  for (int s = 0; s < PO::NREG; ++s) {
    const int rr = PO::nrow(tid, s);
    const int64_t src = rr < rows ? (a.gather ? (int64_t)a.gather[row0 + rr] : row0 + rr) : 0;
    prowp[s] = rr < rows ? Pb + src * a.ldp * ES : nullptr;
  }
  const char* qrowp[QO::NREG];
  const char* qkbase = nullptr;
  int64_t qldk = 0;
  if constexpr (!QT) {
#pragma unroll
    for (int s = 0; s < QO::NREG; ++s) {
      const int q = QO::nrow(tid, s);
      int64_t off;
      if constexpr (OP == OP_GU_FWD) {
        // tile = BN/2 gate rows then the matching BN/2 up rows of one expert block
        const int blk = n0 / a.sub, r0 = n0 - blk * a.sub;
        const int wrow = blk * 2 * a.sub + (q < BN / 2 ? r0 + q : a.sub + r0 + (q - BN / 2));
        off = (int64_t)wrow * a.ldq;
      } else {
        // OP_DOWN_FWD: Q[n][c] = W[c / sub][n][c % sub]; the block part is added per chunk
        off = (int64_t)(n0 + q) * a.sub;
      }
      qrowp[s] = Qb + off * ES;
    }
  } else {
    if constexpr (OP == OP_DOWN_DGRAD) {
      // Q[c][k] = W[c / sub][k][c % sub]; a tile never straddles two blocks
      const int blk = n0 / a.sub, c0 = n0 - blk * a.sub;
      qkbase = Qb + ((int64_t)blk * a.K * a.sub + c0) * ES;
      qldk = (int64_t)a.sub * ES;
    } else {
      qkbase = Qb + (int64_t)n0 * ES;
      qldk = a.ldq * ES;
    }
  }
  auto load = [&](int kc, PO& po, QO& qo) {
    po.load_normal(prowp, (int64_t)kc * ES, tid);
    if constexpr (!QT) {
      int64_t koff = (int64_t)kc * ES;
      if constexpr (OP == OP_DOWN_FWD) {
        const int blk = kc / a.sub, kk = kc - blk * a.sub;
        koff = ((int64_t)blk * a.N * a.sub + kk) * ES;
      }
      qo.load_normal(qrowp, koff, tid);
    } else {
      qo.load_kmajor(qkbase + (int64_t)kc * qldk, qldk, BK, tid);
    }
  };
  auto stage = [&](char* buf, const PO& po, const QO& qo) {
    po.stage_normal(buf, tid);
    if constexpr (!QT) qo.stage_normal(buf + PO::BYTES, tid);
    else qo.stage_kmajor(buf + PO::BYTES, tid);
  };

  PO po;
  QO qo;
  load(0, po, qo);
  stage(smem, po, qo);
  __syncthreads();
  for (int kc = 0; kc < nk; ++kc) {
    const bool more = kc + 1 < nk;
    if (more) load((kc + 1) * BK, po, qo);
    const char* buf = smem + (kc & 1) * STAGE;
    mfma_chunk<T, PO, QO, NS, MS>(acc, buf + PO::BYTES, buf, qrow, prow, lane);
    if (more) stage(smem + ((kc + 1) & 1) * STAGE, po, qo);
    __syncthreads();
  }
  }  // main loops

  if constexpr (PERM) {
    // ---- staged epilogue (16-bit path)
    // LDS barrier without the release fence of __syncthreads(), which would
    // also wait for this wave's outstanding global stores
    auto lds_barrier = [&]() {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };
    auto sp = [&](int arr, int sr, int c) -> char* {
      return smem + arr * SR * RB + sr * RB + ((c ^ (sr & 7)) << 4);
    };
    const int sr_l = wm * 32 + (lane & 31);                   // this lane's staged row
    // MX SwiGLU backward: padded K position of the tile's first row in the
    // token-axis codes of [dG | dU], and the scale bytes of this thread's
    // column for the tile's BM / 32 blocks
    [[maybe_unused]] const int64_t tkbase = (a.tpad ? (int64_t)a.tpad[g] : 0) + (row0 - seg0);
    [[maybe_unused]] uint32_t tsc = 0;
    // their LDS staging: [2 BN][BM] bytes after the staged dG, dU rows
    constexpr int TQ_OFF = NARR * SR * RB;
    static_assert(!(MX && EPI == EPI_SWIGLU_BWD) || TQ_OFF + 2 * BN * BM <= NSTG * (BM + BN) * DKB,
                  "token-axis code staging fits in the ring");
    // (SwiGLU forward: H's, TILE_N columns of BM bytes, then their BM / 32 scale bytes each)
    constexpr int HQ_OFF = NARR * SR * RB;
    static_assert(!(MX && EPI == EPI_SWIGLU_FWD) || HQ_OFF + TILE_N * (BM + BM / 32) <= NSTG * (BM + BN) * DKB,
                  "token-axis code staging fits in the ring");
    // f32 G, U of the SwiGLU backward: this lane's row pieces of column
    // subtile ns, loaded one subtile ahead of the one being computed; in
    // ping-pong tiles also the next pass's first subtile during this pass's
    // last one (NS is even, so that subtile computes from gub[1] while gub[0]
    // fills; the smaller tiles would spill the registers it keeps live)
    constexpr bool GU_DIRECT = GUF32 && EPI == EPI_SWIGLU_BWD;
    static_assert(!GU_DIRECT || NS % 2 == 0, "G/U double buffer alternates over an even subtile count");
    float gub[2][GU_DIRECT ? NRUN : 1][2][RUN];
    auto load_gu_f32 = [&](float (&dst)[GU_DIRECT ? NRUN : 1][2][RUN], int trow, int ns) {
      if constexpr (GU_DIRECT) {
#pragma unroll
        for (int t = 0; t < NRUN; ++t) {
          const int c = (qrow[ns] + RSTEP * t + RUN * h) / 8;
          const float* gp = static_cast<const float*>(a.aux) + (row0 + (trow < rows ? trow : 0)) * a.ldaux +
                            gcol0 + c * 8;
          load4<float>(gp, dst[t][0]);
          load4<float>(gp + 4, dst[t][0] + 4);
          load4<float>(gp + a.sub, dst[t][1]);
          load4<float>(gp + a.sub + 4, dst[t][1] + 4);
        }
      }
    };
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
      lds_barrier();                                          // ring / previous pass no longer read
      // this lane's tile row in the pass (MFMA layout) and, for the SwiGLU
      // backward of routed experts, its routing weight and g partial
      const int tr_l = prow[ms] + (lane & 31);
      float wrow_l = 1.0f;
      // partial sums of (P Q) * H per column subtile and run, added in order after the loop
      float gpiece[EPI == EPI_SWIGLU_BWD ? NS : 1][EPI == EPI_SWIGLU_BWD ? NRUN : 1];
      if constexpr (EPI == EPI_SWIGLU_BWD) {
        if (a.wrow && tr_l < rows) wrow_l = a.wrow[row0 + tr_l];
      }
      if constexpr (EPI == EPI_SWIGLU_BWD && !GUF32) {
        if constexpr (GU_PRE || GU_PIPE) {
          if constexpr (GU_PIPE) {
            if (ms == 0 && !gu_first) load_gu_rows(gun, 0);
          }
#pragma unroll
          for (int i = 0; i < SITER; ++i) {
            const int q = tid + 64 * NW * i, sr = q / CPR, c = q % CPR;
            st16(sp(0, sr, c), gun[0][i]);
            st16(sp(1, sr, c), gun[1][i]);
          }
          if (ms + 1 < MS) load_gu_rows(gun, ms + 1);
        } else {
          u32x4 cur[2][SITER];
          load_gu_rows(cur, ms);
#pragma unroll
          for (int i = 0; i < SITER; ++i) {
            const int q = tid + 64 * NW * i, sr = q / CPR, c = q % CPR;
            st16(sp(0, sr, c), cur[0][i]);
            st16(sp(1, sr, c), cur[1][i]);
          }
        }
        lds_barrier();
      }
      if constexpr (GU_DIRECT) {
        if (ms == 0 || !PP) load_gu_f32(gub[0], tr_l, 0);
      }
      // accumulators -> staging (MFMA layout: 8 consecutive columns per run)
#pragma unroll
      for (int ns = 0; ns < NS; ++ns) {
        if constexpr (EPI == EPI_SWIGLU_FWD) {
          if (ns >= NS / 2) continue;
        }
        if constexpr (EPI == EPI_SWIGLU_BWD) {
          // one column subtile at a time: its G/U reads (LDS or, f32, global
          // one subtile ahead) are not hoisted above the previous subtile
          asm volatile("" ::: "memory");
          if constexpr (GU_DIRECT) {
            if (ns + 1 < NS) load_gu_f32(gub[(ns + 1) & 1], tr_l, ns + 1);
            else if (PP && ms + 1 < MS) load_gu_f32(gub[0], prow[ms + 1] + (lane & 31), 0);
          }
        }
#pragma unroll
        for (int t = 0; t < NRUN; ++t) {
          float v[RUN];
#pragma unroll
          for (int i = 0; i < RUN; ++i) v[i] = acc[ns][ms][RUN * t + i];
          if constexpr (EPI == EPI_STORE) {
            const int c = (qrow[ns] + RSTEP * t + RUN * h) / 8;
            store8<TO>(reinterpret_cast<TO*>(sp(0, sr_l, c)), v);
          } else if constexpr (EPI == EPI_STORE_F32) {
            const int c = (qrow[ns] + RSTEP * t + RUN * h) / 4;
            store4<float>(reinterpret_cast<float*>(sp(0, sr_l, c)), v[0], v[1], v[2], v[3]);
            store4<float>(reinterpret_cast<float*>(sp(0, sr_l, c + 1)), v[4], v[5], v[6], v[7]);
          } else if constexpr (EPI == EPI_SWIGLU_FWD) {
            // gate subtile ns pairs with up subtile ns + NS/2 (same H columns)
            const int c = (wn * (WTN / 2) + ns * 32 + RSTEP * t + RUN * h) / 8;
            float uv[RUN], hv[RUN];
#pragma unroll
            for (int i = 0; i < RUN; ++i) {
              uv[i] = acc[ns + NS / 2][ms][RUN * t + i];
              hv[i] = silu_f(v[i]) * uv[i];
            }
            if constexpr (GUF32) {
              // G and U in f32 straight from the accumulators (lanes l and
              // l + 32 write the two halves of a 64-byte row piece)
              if (tr_l < rows) {
                float* gp = reinterpret_cast<float*>(a.C) + (row0 + tr_l) * a.ldc + gcol0 + c * 8;
                store4<float>(gp, v[0], v[1], v[2], v[3]);
                store4<float>(gp + 4, v[4], v[5], v[6], v[7]);
                store4<float>(gp + a.sub, uv[0], uv[1], uv[2], uv[3]);
                store4<float>(gp + a.sub + 4, uv[4], uv[5], uv[6], uv[7]);
              }
            } else {
              store8<TO>(reinterpret_cast<TO*>(sp(0, sr_l, c)), v);
              store8<TO>(reinterpret_cast<TO*>(sp(1, sr_l, c)), uv);
            }
            store8<TO>(reinterpret_cast<TO*>(sp(2, sr_l, c)), hv);
          } else if constexpr (EPI == EPI_SWIGLU_BWD) {
            // v = (P Q) row piece, dH = wrow * v; G, U staged at the same
            // positions (f32 G, U: loaded here), overwritten by dG, dU
            const int c = (qrow[ns] + RSTEP * t + RUN * h) / 8;
            float G[RUN], U[RUN];
            if constexpr (GUF32) {
#pragma unroll
              for (int i = 0; i < RUN; ++i) {
                G[i] = gub[ns & 1][t][0][i];
                U[i] = gub[ns & 1][t][1][i];
              }
            } else {
              unpack8<TO>(ld16(sp(0, sr_l, c)), G);
              unpack8<TO>(ld16(sp(1, sr_l, c)), U);
            }
            // dG, dU with the routing weight applied last (it does not
            // depend on G, U: applied first, the products would be formed
            // early and held); then w H, formed after dG, dU are stored
            float gl = 0.0f, dG[RUN], dU[RUN];
#pragma unroll
            for (int i = 0; i < RUN; ++i) {
              const float sg = sigmoid_f(G[i]);
              const float dU0 = v[i] * G[i] * sg;
              const float dG0 = v[i] * U[i] * sg * (1.0f + G[i] * (1.0f - sg));
              gl = fmaf(dU0, U[i], gl);
              dG[i] = wrow_l * dG0;
              dU[i] = wrow_l * dU0;
            }
            gpiece[ns][t] = gl;
            store8<TO>(reinterpret_cast<TO*>(sp(0, sr_l, c)), dG);
            store8<TO>(reinterpret_cast<TO*>(sp(1, sr_l, c)), dU);
            if constexpr (LO) {
              // rounding remainders of dG, dU, straight from registers
              if (tr_l < rows) {
                TO* dst = static_cast<TO*>(a.C_lo) + (row0 + tr_l) * a.ldc + gcol0 + c * 8;
#pragma unroll
                for (int i = 0; i < RUN; ++i) {
                  dG[i] -= to_f32<TO>(from_f32<TO>(dG[i]));
                  dU[i] -= to_f32<TO>(from_f32<TO>(dU[i]));
                }
                store8<TO>(dst, dG);
                store8<TO>(dst + a.sub, dU);
              }
            }
            if constexpr (WH) {
              if (a.C2) {
                asm volatile("" ::: "memory");
                float wh[RUN];
#pragma unroll
                for (int i = 0; i < RUN; ++i) wh[i] = wrow_l * (silu_f(G[i]) * U[i]);
                if constexpr (WH_STAGED) store8<TO>(reinterpret_cast<TO*>(sp(2, sr_l, c)), wh);
                else if (tr_l < rows) store8<TO>(static_cast<TO*>(a.C2) + (row0 + tr_l) * a.ldc2 + n0 + c * 8, wh);
                if constexpr (LO) {
                  if (tr_l < rows) {
#pragma unroll
                    for (int i = 0; i < RUN; ++i) wh[i] -= to_f32<TO>(from_f32<TO>(wh[i]));
                    store8<TO>(static_cast<TO*>(a.C2_lo) + (row0 + tr_l) * a.ldc2 + n0 + c * 8, wh);
                  }
                }
              }
            }
          }
        }
      }
      if constexpr (EPI == EPI_SWIGLU_BWD) {
        if (a.gpart) {
          float gacc = 0.0f;
#pragma unroll
          for (int ns = 0; ns < NS; ++ns)
#pragma unroll
            for (int t = 0; t < NRUN; ++t) gacc += gpiece[ns][t];
          // lanes l and l + 32 hold the two column halves of row l % 32
          const float gs = gacc + __shfl_xor(gacc, 32, 64);
          if (h == 0 && tr_l < rows) a.gpart[(row0 + tr_l) * a.gparts + (n0 / BN) * WN + wn] = gs;
        }
      }
      lds_barrier();
      // staging -> global, whole rows
#pragma unroll
      for (int i = 0; i < SITER; ++i) {
        const int q = tid + 64 * NW * i, sr = q / CPR, c = q % CPR;
        const int tr = srow(sr, ms);
        if (tr >= rows) continue;
        const int64_t row = row0 + tr;
        if constexpr (EPI == EPI_STORE) {
          st16(static_cast<TO*>(a.C) + row * a.ldc + n0 + c * 8, ld16(sp(0, sr, c)));
        } else if constexpr (EPI == EPI_STORE_F32) {
          st16(static_cast<float*>(a.C) + row * a.ldc + n0 + c * 4, ld16(sp(0, sr, c)));
        } else if constexpr (EPI == EPI_SWIGLU_FWD) {
          if constexpr (!GUF32) {
            TO* gu = static_cast<TO*>(a.C) + row * a.ldc + gcol0 + c * 8;
            st16(gu, ld16(sp(0, sr, c)));
            st16(gu + a.sub, ld16(sp(1, sr, c)));
          }
          const u32x4 hraw = ld16(sp(2, sr, c));
          // (MX with H's token-axis codes: the act-dtype H rows only if C2 is given)
          if (!MX || a.C2) st16(static_cast<TO*>(a.C2) + row * a.ldc2 + n0 + c * 8, hraw);
          if constexpr (MX) {
            // the stored H row-wise in MX-fp8 for the down projection: the
            // four lanes of chunks 4b .. 4b+3 (one row, consecutive lanes)
            // hold a 32-column block
            if (a.Hq) {
              float hv[8];
              unpack8<TO>(hraw, hv);
              float amax = 0.0f;
#pragma unroll
              for (int q = 0; q < 8; ++q) amax = fmaxf(amax, fabsf(hv[q]));
              amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
              amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
              const int x = mx_scale_exp(amax);
              const float sc = ldexpf(1.0f, -x);
              const u32x2 o = {e4m3x4(hv[0], hv[1], hv[2], hv[3], sc), e4m3x4(hv[4], hv[5], hv[6], hv[7], sc)};
              st8(a.Hq + row * a.ldc2 + n0 + c * 8, o);
              if ((c & 3) == 0) a.Hs[row * (a.ldc2 / 32) + (n0 + c * 8) / 32] = (uint8_t)(x + 127);
            }
          }
        } else if constexpr (EPI == EPI_SWIGLU_BWD) {
          const u32x4 dgraw = ld16(sp(0, sr, c)), duraw = ld16(sp(1, sr, c));
          // (MX: the act-dtype [dG | dU] only on request, C non-null)
          if (!MX || a.C) {
            TO* dgu = static_cast<TO*>(a.C) + row * a.ldc + gcol0 + c * 8;
            st16(dgu, dgraw);
            st16(dgu + a.sub, duraw);
          }
          if constexpr (WH_STAGED) {
            if (a.C2) st16(static_cast<TO*>(a.C2) + row * a.ldc2 + n0 + c * 8, ld16(sp(2, sr, c)));
          }
          if constexpr (MX) {
            // [dG | dU] row-wise in MX-fp8 for the gate/up dgrad: four
            // consecutive lanes hold a 32-column block of each half
            if (a.Hq) {
#pragma unroll
              for (int half = 0; half < 2; ++half) {
                float v8[8];
                unpack8<TO>(half ? duraw : dgraw, v8);
                float amax = 0.0f;
#pragma unroll
                for (int q = 0; q < 8; ++q) amax = fmaxf(amax, fabsf(v8[q]));
                amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
                amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
                const int x = mx_scale_exp(amax);
                const float sc = ldexpf(1.0f, -x);
                const u32x2 o = {e4m3x4(v8[0], v8[1], v8[2], v8[3], sc), e4m3x4(v8[4], v8[5], v8[6], v8[7], sc)};
                const int64_t col = gcol0 + c * 8 + half * a.sub;
                st8(a.Hq + row * a.ldc + col, o);
                if ((c & 3) == 0) a.Hs[row * (a.ldc / 32) + col / 32] = (uint8_t)(x + 127);
              }
            }
          }
        }
      }
      if constexpr (MX && EPI == EPI_SWIGLU_FWD) {
        // H along the tokens for the down weight gradient (optional, saved
        // beside H): thread j < WM * TILE_N takes H column j % TILE_N of the
        // tile and the pass's staged 32-row block j / TILE_N (tile rows
        // gi WTM + 32 ms ..).  The tile starts a 32-block of its segment and
        // rows past the segment were staged as zeros (their P rows read as
        // zero), as the padding they stand for.  The codes wait in LDS (after
        // the staged rows: column j's BM bytes at HQ_OFF + j BM, 16-byte
        // chunk q at (q ^ (j & 7)), then its BM / 32 scale bytes) until the
        // tile is whole.
        if (a.Tq) {
          static_assert(64 * NW >= WM * TILE_N, "a thread per (column, row block)");
          const int col = tid % TILE_N, gi = tid / TILE_N;
          const int tb = gi * WTM + ms * 32;
          if (gi < WM) {
            float v[32];
#pragma unroll
            for (int r = 0; r < 32; ++r)
              v[r] = to_f32<TO>(reinterpret_cast<const TO*>(sp(2, gi * 32 + r, col / 8))[col % 8]);
            float amax = 0.0f;
#pragma unroll
            for (int r = 0; r < 32; ++r) amax = fmaxf(amax, fabsf(v[r]));
            const int x = mx_scale_exp(amax);
            const float sc = ldexpf(1.0f, -x);
            u32x4 o[2];
#pragma unroll
            for (int w = 0; w < 8; ++w) o[w >> 2][w & 3] = e4m3x4(v[4 * w], v[4 * w + 1], v[4 * w + 2], v[4 * w + 3], sc);
            uint8_t* crow = reinterpret_cast<uint8_t*>(smem) + HQ_OFF + col * BM;
            const int q0 = tb / 16;
            *reinterpret_cast<u32x4*>(crow + ((q0 ^ (col & 7)) << 4)) = o[0];
            *reinterpret_cast<u32x4*>(crow + (((q0 + 1) ^ (col & 7)) << 4)) = o[1];
            reinterpret_cast<uint8_t*>(smem)[HQ_OFF + TILE_N * BM + col * (BM / 32) + tb / 32] = (uint8_t)(x + 127);
          }
        }
      }
      if constexpr (MX && EPI == EPI_SWIGLU_BWD) {
        // [dG | dU] along the tokens for the gate/up weight gradient: thread
        // j takes column j of the tile's [dG | dU] and quantises the pass's WM
        // staged blocks of 32 rows (tile rows gi WTM + 32 ms ..; the tile
        // starts a 32-block of its segment, and rows past the segment were
        // staged as zeros, as the padding they stand for)
        if (a.Tq) {
          static_assert(64 * NW == 2 * BN, "one thread per column of [dG | dU]");
          const int arr = tid / BN, col = tid % BN;
          // the codes wait in LDS (the free half of the ring), row j = column
          // j, 16-byte chunk q at (q ^ (j & 7)), until the tile's rows are
          // whole; then every row leaves as one 128-byte store
          uint8_t* crow = reinterpret_cast<uint8_t*>(smem) + TQ_OFF + tid * BM;
#pragma unroll
          for (int gi = 0; gi < WM; ++gi) {
            float v[32];
#pragma unroll
            for (int r = 0; r < 32; ++r)
              v[r] = to_f32<TO>(reinterpret_cast<const TO*>(sp(arr, gi * 32 + r, col / 8))[col % 8]);
            float amax = 0.0f;
#pragma unroll
            for (int r = 0; r < 32; ++r) amax = fmaxf(amax, fabsf(v[r]));
            const int x = mx_scale_exp(amax);
            const float sc = ldexpf(1.0f, -x);
            u32x4 o[2];
#pragma unroll
            for (int w = 0; w < 8; ++w) o[w >> 2][w & 3] = e4m3x4(v[4 * w], v[4 * w + 1], v[4 * w + 2], v[4 * w + 3], sc);
            const int tb = gi * WTM + ms * 32, q0 = tb / 16;
            *reinterpret_cast<u32x4*>(crow + ((q0 ^ (tid & 7)) << 4)) = o[0];
            *reinterpret_cast<u32x4*>(crow + (((q0 + 1) ^ (tid & 7)) << 4)) = o[1];
            tsc |= (uint32_t)(x + 127) << (8 * (tb / 32));
          }
        }
      }
    }
    if constexpr (MX && EPI == EPI_SWIGLU_FWD) {
      // the tile's H codes: each column's rows up to the segment's 128-padded
      // end (the last 256-row tile of a segment stops there), 16 bytes per
      // thread, and its scale bytes as 4-byte words
      if (a.Tq) {
        lds_barrier();                                        // every column's codes staged
        const int tq_rows = (rows + 127) / 128 * 128;
        const uint8_t* cst = reinterpret_cast<const uint8_t*>(smem) + HQ_OFF;
        constexpr int CH = BM / 16;                           // 16-byte chunks per column
#pragma unroll
        for (int i = 0; i < (TILE_N * CH + 64 * NW - 1) / (64 * NW); ++i) {
          const int q = tid + 64 * NW * i, j = q / CH, ch = q % CH;
          if (j < TILE_N && ch * 16 < tq_rows)
            st16(a.Tq + (int64_t)(n0 + j) * a.ldt + tkbase + ch * 16,
                 *reinterpret_cast<const u32x4*>(cst + j * BM + ((ch ^ (j & 7)) << 4)));
        }
        constexpr int SW = BM / 128;                          // 4-byte scale words per column
        if (tid < TILE_N * SW) {
          const int j = tid / SW, w = tid % SW;
          if (w * 128 < tq_rows)
            *reinterpret_cast<uint32_t*>(a.Ts + (int64_t)(n0 + j) * (a.ldt / 32) + tkbase / 32 + 4 * w) =
                *reinterpret_cast<const uint32_t*>(cst + TILE_N * BM + j * (BM / 32) + 4 * w);
        }
      }
    }
    if constexpr (MX && EPI == EPI_SWIGLU_BWD) {
      if (a.Tq) {
        static_assert(BM == 128, "four token blocks per tile: 128 code bytes and one 4-byte scale store per column");
        const int arr = tid / BN, col = tid % BN;
        *reinterpret_cast<uint32_t*>(a.Ts + (gcol0 + col + arr * a.sub) * (a.ldt / 32) + tkbase / 32) = tsc;
        lds_barrier();                                        // every column's codes staged
        const uint8_t* cst = reinterpret_cast<const uint8_t*>(smem) + TQ_OFF;
#pragma unroll
        for (int i = 0; i < 2 * BN * (BM / 16) / (64 * NW); ++i) {
          const int q = tid + 64 * NW * i, j = q >> 3, ch = q & 7;
          const int jarr = j / BN, jcol = j % BN;
          st16(a.Tq + (gcol0 + jcol + jarr * a.sub) * a.ldt + tkbase + ch * 16,
               *reinterpret_cast<const u32x4*>(cst + j * BM + ((ch ^ (j & 7)) << 4)));
        }
      }
    }
  } else {
  // ---- direct epilogue (f32 path): accumulator [ns][ms] holds row prow[ms] + lane%32
#pragma unroll
  for (int ms = 0; ms < MS; ++ms) {
    const int ml = prow[ms] + (lane & 31);
    const bool live = ml < rows;
    const int64_t row = row0 + (live ? ml : 0);
    if constexpr (EPI == EPI_SWIGLU_BWD) {
      // routed experts: dH = wrow * (P Q) and the partial row sums of
      // (P Q) * H over this wave's columns (lanes l, l + 32 share a row)
      const float wr = (a.wrow && live) ? a.wrow[row] : 1.0f;
      float gacc = 0.0f;
#pragma unroll
      for (int ns = 0; ns < NS; ++ns)
#pragma unroll
        for (int t = 0; t < NRUN; ++t) {
          const int n = n0 + qrow[ns] + RSTEP * t + RUN * h;
          const int blk = n / a.sub;
          const int gcol = blk * 2 * a.sub + (n - blk * a.sub);
          float G[RUN], U[RUN], dG[RUN], dU[RUN], wh[RUN];
          const T* gu = static_cast<const T*>(a.aux) + row * a.ldaux;
          load_run<T, RUN>(gu + gcol, G);
          load_run<T, RUN>(gu + gcol + a.sub, U);
#pragma unroll
          for (int i = 0; i < RUN; ++i) {
            const float vv = acc[ns][ms][RUN * t + i];
            const float sg = sigmoid_f(G[i]);
            const float gs = G[i] * sg;
            const float dU0 = vv * gs;
            const float dG0 = vv * U[i] * sg * (1.0f + G[i] * (1.0f - sg));
            gacc = fmaf(dU0, U[i], gacc);
            dG[i] = wr * dG0;
            dU[i] = wr * dU0;
            wh[i] = wr * (gs * U[i]);
          }
          if (live) {
            T* dgu = static_cast<T*>(a.C) + row * a.ldc;
            store_run<T, RUN>(dgu + gcol, dG);
            store_run<T, RUN>(dgu + gcol + a.sub, dU);
            if (a.C2) store_run<T, RUN>(static_cast<T*>(a.C2) + row * a.ldc2 + n, wh);
          }
        }
      if (a.gpart) {
        const float gs = gacc + __shfl_xor(gacc, 32, 64);
        if (h == 0 && live) a.gpart[row * a.gparts + (n0 / BN) * WN + wn] = gs;
      }
      continue;
    }
    if (!live) continue;
    if constexpr (EPI == EPI_SWIGLU_FWD) {
#pragma unroll
      for (int j = 0; j < NS / 2; ++j)
#pragma unroll
        for (int t = 0; t < NRUN; ++t) {
          const int hc = n0 + wn * (WTN / 2) + j * 32 + RSTEP * t + RUN * h;
          const int blk = hc / a.sub;
          const int gcol = blk * 2 * a.sub + (hc - blk * a.sub);
          float gv[RUN], uv[RUN], hv[RUN];
#pragma unroll
          for (int i = 0; i < RUN; ++i) {
            gv[i] = acc[j][ms][RUN * t + i];
            uv[i] = acc[j + NS / 2][ms][RUN * t + i];
            hv[i] = silu_f(gv[i]) * uv[i];
          }
          T* gu = static_cast<T*>(a.C) + row * a.ldc;
          store_run<T, RUN>(gu + gcol, gv);
          store_run<T, RUN>(gu + gcol + a.sub, uv);
          store_run<T, RUN>(static_cast<T*>(a.C2) + row * a.ldc2 + hc, hv);
        }
    } else {
#pragma unroll
      for (int ns = 0; ns < NS; ++ns)
#pragma unroll
        for (int t = 0; t < NRUN; ++t) {
          const int n = n0 + qrow[ns] + RSTEP * t + RUN * h;
          float v[RUN];
#pragma unroll
          for (int i = 0; i < RUN; ++i) v[i] = acc[ns][ms][RUN * t + i];
          if constexpr (EPI == EPI_STORE) {
            store_run<T, RUN>(static_cast<T*>(a.C) + row * a.ldc + n, v);
          } else if constexpr (EPI == EPI_STORE_F32) {
            store_run<float, RUN>(static_cast<float*>(a.C) + row * a.ldc + n, v);
          }
        }
    }
  }
  }
}

// ------------------------------------------------------------- wgrad GEMM ---
// MX: P is [M][Kpad] and Q [N][Kpad] MX-fp8 payload bytes (token axis
// contiguous, segments at the padded offsets in a.offsets, each a multiple of
// 128 tokens, zero past the segment's tokens), scales a.Ps / a.Qs; outputs bf16
// (or f32 partials).
template <typename T, int BM, int BN, int OUT_F32, int WM, int WN, bool MX = false, bool PP = false>
__device__ __forceinline__ void wgrad_body(const WgradArgs& a, char* smem) {
  constexpr int ES = sizeof(T);
  static_assert(!PP || (ES == 2 && BM == 256 && BN == 256 && WM == 2 && WN == 4), "ping-pong tile");
  using TO = std::conditional_t<MX, __bf16, T>;
  constexpr int NW = WM * WN;
  static_assert(ES == 2 || MX || NW == 4, "the register-staged path runs 4 waves");
  static_assert(!MX || (ES == 1 && ((BM == 128 && BN == 128 && NW == 4) || (BM == 256 && BN == 256 && NW == 8))),
                "MX weight-gradient tiles: 128 x 128 with 4 waves or 256 x 256 with 8");
  using TOP = std::conditional_t<MX, __bf16, T>;
  using PO = Operand<TOP, BM, true>;
  using QO = Operand<TOP, BN, true>;
  constexpr int BK = MX ? MX_DKB : PO::BK;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MS = WTM / 32, NS = WTN / 32;
  constexpr int STAGE = PO::BYTES + QO::BYTES;

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int n_mt = a.M / BM, n_nt = a.N / BN;
  // Tile order.  Segments of similar length: each XCD takes a contiguous run
  // of tiles (whole experts, so an expert's operand slices are read into one
  // L2).  Skewed segments (the longest over twice the mean): chunks of the n
  // tiles of one (expert, split, m tile), which share its P slice, dealt
  // round-robin over the XCDs, so the busiest experts do not all land on one
  // XCD.  Every wave derives the same choice from the offsets.
  bool skewed = false;
  if (a.offsets && a.G > 1) {
    int mx = 0, tot = 0;
    for (int gg = lane; gg < a.G; gg += 64) {
      const int len = a.offsets[gg + 1] - a.offsets[gg];
      mx = len > mx ? len : mx;
      tot += len;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const int m2 = __shfl_xor(mx, o, 64);
      mx = m2 > mx ? m2 : mx;
      tot += __shfl_xor(tot, o, 64);
    }
    // every lane holds the totals: read them as scalars, so the tile indices
    // (and the buffer descriptors built from them) stay wave-uniform values
    mx = __builtin_amdgcn_readfirstlane(mx);
    tot = __builtin_amdgcn_readfirstlane(tot);
    skewed = (int64_t)mx * a.G > 2 * (int64_t)tot;
  }
  const int ntiles = a.G * a.splits * n_mt * n_nt;
  const int logical = skewed ? xcd_chunked(blockIdx.x, ntiles, n_nt) : xcd_logical(blockIdx.x, ntiles);
  if (logical < 0) return;
  int rest = logical;
  const int nt = rest % n_nt; rest /= n_nt;
  const int mt = rest % n_mt; rest /= n_mt;
  const int sp = rest % a.splits;
  const int g = rest / a.splits;

  const int64_t s0 = a.offsets ? a.offsets[g] : 0;
  const int64_t s1 = a.offsets ? a.offsets[g + 1] : a.Mtok;
  const int64_t nchunk = (s1 - s0 + BK - 1) / BK;
  const int64_t per = (nchunk + a.splits - 1) / a.splits;
  const int64_t kbeg = s0 + sp * per * BK;
  int64_t kend = kbeg + per * BK;
  if (kend > s1) kend = s1;
  const int nk = kend > kbeg ? (int)((kend - kbeg + BK - 1) / BK) : 0;
  const int m0 = mt * BM, n0 = nt * BN;

  const char* Pb = static_cast<const char*>(a.P) + (MX ? 0 : (int64_t)m0 * ES);
  const char* Qb = static_cast<const char*>(a.Q) + (MX ? 0 : (int64_t)n0 * ES);
  const int64_t pld = a.ldp * ES, qld = a.ldq * ES;
  // ping-pong: group wave / 4 owns a row half, its four waves (one per SIMD) the column quarters
  const int wm = PP ? wave / WN : wave % WM, wn = PP ? wave % WN : wave / WM;
  int qrow[NS], prow[MS];
#pragma unroll
  for (int ns = 0; ns < NS; ++ns) qrow[ns] = wn * WTN + ns * 32;
#pragma unroll
  for (int ms = 0; ms < MS; ++ms) prow[ms] = wm * WTM + ms * 32;
  f32x16 acc[NS][MS];
  zero_acc(acc);

  if constexpr (MX) {
    // rows m0.. of P and n0.. of Q, each K-contiguous; chunk = 128 tokens
    constexpr int NSTG = 2;
    using PD = DmaRows<BM, NW, MX_DKB>;
    using QD = DmaRows<BN, NW, MX_DKB>;
    constexpr int DSTAGE = PD::BYTES + QD::BYTES;
    constexpr int SSTAGE = (BM + BN) * 4;
    constexpr int SC_OFF = NSTG * DSTAGE;
    const int64_t pls = a.ldp / 32, qls = a.ldq / 32;
    uint32_t poff[PD::NI], qoff[QD::NI];
#pragma unroll
    for (int s2 = 0; s2 < PD::NI; ++s2) {
      const int r = PD::row_of(wave, s2, lane);
      poff[s2] = (uint32_t)(r * a.ldp + PD::gchunk(r, lane) * 16);
    }
#pragma unroll
    for (int s2 = 0; s2 < QD::NI; ++s2) {
      const int r = QD::row_of(wave, s2, lane);
      qoff[s2] = (uint32_t)(r * a.ldq + QD::gchunk(r, lane) * 16);
    }
    // scale rows: the first BM / 64 waves load P's rows 64 w .., the others Q's
    static_assert(64 * NW == BM + BN, "one wave per 64 scale rows");
    const bool sq_side = wave >= BM / 64;
    const int swave = sq_side ? wave - BM / 64 : wave;
    const int sr = swave * 64 + lane;
    const uint32_t soff = sq_side ? (uint32_t)((n0 + sr) * qls) : (uint32_t)((m0 + sr) * pls);
    const uint8_t* sbase = sq_side ? a.Qs : a.Ps;
    const int64_t ldp = a.ldp, ldq = a.ldq;
    auto issue = [&](int64_t kc, int st) {
      char* stage = smem + st * DSTAGE;
      const rsrc_t prs = make_rsrc(Pb + (int64_t)m0 * ldp + kc, 0x7fffffffu);
      const rsrc_t qrs = make_rsrc(Qb + (int64_t)n0 * ldq + kc, 0x7fffffffu);
#pragma unroll
      for (int s2 = 0; s2 < PD::NI; ++s2) dma16(prs, stage + PD::lds_off(wave, s2), poff[s2]);
#pragma unroll
      for (int s2 = 0; s2 < QD::NI; ++s2) dma16(qrs, stage + PD::BYTES + QD::lds_off(wave, s2), qoff[s2]);
      char* sst = smem + SC_OFF + st * SSTAGE + (sq_side ? BM * 4 : 0) + swave * 64 * 4;
      dma4(make_rsrc(sbase + kc / 32, 0x7fffffffu), sst, soff);
    };
    constexpr int LPC = PD::NI + QD::NI + 1;
    const int nkd = nk;
#pragma unroll
    for (int c = 0; c < NSTG - 1; ++c)
      if (c < nkd) issue(kbeg + (int64_t)c * MX_DKB, c);
    for (int kc = 0; kc < nkd; ++kc) {
      ring_barrier<LPC, NSTG>(nkd - 1 - kc);
      if (kc + NSTG - 1 < nkd) issue(kbeg + (int64_t)(kc + NSTG - 1) * MX_DKB, (kc + NSTG - 1) % NSTG);
      const int st = kc % NSTG;
      const char* buf = smem + st * DSTAGE;
      const uint8_t* sbuf = reinterpret_cast<const uint8_t*>(smem + SC_OFF + st * SSTAGE);
      mfma_chunk_mx<NS, MS>(acc, buf + PD::BYTES, buf, sbuf + BM * 4, sbuf, qrow, prow, lane);
    }
  } else if constexpr (ES == 2 && PP) {
    // ---------------- ping-pong main loop (see the row GEMM's): group 0
    // streams P's token chunks, group 1 Q's; chunk = 32 tokens of the split
    constexpr int DKB = TileCfg<BM, BN, true, true>::DKB, NSTG = TileCfg<BM, BN, true, true>::NSTG;
    constexpr int NWL = 4;
    using PD = DmaKmajor<BM, NWL, DKB>;
    using QD = DmaKmajor<BN, NWL, DKB>;
    static_assert(PD::NI == QD::NI, "both halves issue the same number of loads per wave");
    constexpr int DSTAGE = PD::BYTES + QD::BYTES;
    constexpr int KSTEPS = DKB / 32;
    constexpr int LPH = PD::NI;
    constexpr int DBKK = PD::KROWS;                   // tokens per chunk
    const int grp = wave >> 2, wq = wave & 3;
    const char* base = grp == 0 ? Pb : Qb;
    const int64_t ld = grp == 0 ? pld : qld;
    uint32_t off[LPH];
#pragma unroll
    for (int s2 = 0; s2 < LPH; ++s2) {
      const int k = PD::k_of(wq, s2, lane);          // (both halves have the same k-row geometry)
      off[s2] = (uint32_t)(k * ld + PD::gchunk(k, lane) * 16);
    }
    // this wave's half of chunk c; tokens at or past kend read as zero
    auto issue_half = [&](int c) {
      char* stage = smem + (c % NSTG) * DSTAGE + (grp == 0 ? 0 : PD::BYTES);
      const int64_t kc = kbeg + (int64_t)c * DBKK;
      const int kvalid = (int)((kend - kc) < DBKK ? (kend - kc) : DBKK);
      const rsrc_t rs = make_rsrc(base + kc * ld, (uint32_t)(kvalid * ld));
#pragma unroll
      for (int s2 = 0; s2 < LPH; ++s2) dma16(rs, stage + PD::lds_off(wq, s2), off[s2]);
    };
    auto wait_chunk = [&](int c, int nkd) {
      const int later = (nkd - 1 - c) < NSTG - 2 ? (nkd - 1 - c) : NSTG - 2;
      asm volatile("" ::: "memory");
      if (later >= 2) wait_vmcnt<2 * LPH>();
      else if (later == 1) wait_vmcnt<LPH>();
      else wait_vmcnt<0>();
    };
    auto phase_barrier = [&]() {
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };
    static_assert(NSTG - 2 <= 2, "wait_chunk covers at most two later chunks");
    const int nkd = kend > kbeg ? (int)((kend - kbeg + DBKK - 1) / DBKK) : 0;
#pragma unroll
    for (int c = 0; c < NSTG - 1; ++c)
      if (c < nkd) issue_half(c);
    if (nkd > 0) wait_chunk(0, nkd);
    phase_barrier();
    if (grp == 1) phase_barrier();                  // one phase behind group 0
    u32x4 fa[KSTEPS][NS], fb[KSTEPS][MS];
    for (int c = 0; c < nkd; ++c) {
      const char* buf = smem + (c % NSTG) * DSTAGE;
      read_chunk_frags<PD, QD, NS, MS, KSTEPS>(fa, fb, buf + PD::BYTES, buf, qrow, prow, lane);
      if (c + NSTG - 1 < nkd) issue_half(c + NSTG - 1);
      __builtin_amdgcn_s_waitcnt(0xC07F);           // lgkmcnt(0): fragments in registers, slot read
      if (c + 1 < nkd) wait_chunk(c + 1, nkd);
      phase_barrier();
      __builtin_amdgcn_s_setprio(1);
      mfma_chunk_frags<T, NS, MS, KSTEPS>(acc, fa, fb);
      __builtin_amdgcn_s_setprio(0);
      phase_barrier();
    }
    if (grp == 0) phase_barrier();                  // as many barriers as group 1
  } else if constexpr (ES == 2) {
    constexpr int DKB = TileCfg<BM, BN, true>::DKB, NSTG = TileCfg<BM, BN, true>::NSTG;
    using PD = DmaKmajor<BM, NW, DKB>;
    using QD = DmaKmajor<BN, NW, DKB>;
    constexpr int DSTAGE = PD::BYTES + QD::BYTES;
    uint32_t poff[PD::NI], qoff[QD::NI];
#pragma unroll
    for (int s2 = 0; s2 < PD::NI; ++s2) {
      const int k = PD::k_of(wave, s2, lane);
      poff[s2] = (uint32_t)(k * pld + PD::gchunk(k, lane) * 16);
    }
#pragma unroll
    for (int s2 = 0; s2 < QD::NI; ++s2) {
      const int k = QD::k_of(wave, s2, lane);
      qoff[s2] = (uint32_t)(k * qld + QD::gchunk(k, lane) * 16);
    }
    // tokens at or past kend fall outside the per-chunk descriptors and read as zero
    auto issue = [&](int64_t kc, char* stage) {
      const int kvalid = (int)((kend - kc) < PD::KROWS ? (kend - kc) : PD::KROWS);
      const rsrc_t prs = make_rsrc(Pb + kc * pld, (uint32_t)(kvalid * pld));
      const rsrc_t qrs = make_rsrc(Qb + kc * qld, (uint32_t)(kvalid * qld));
#pragma unroll
      for (int s2 = 0; s2 < PD::NI; ++s2) dma16(prs, stage + PD::lds_off(wave, s2), poff[s2]);
#pragma unroll
      for (int s2 = 0; s2 < QD::NI; ++s2) dma16(qrs, stage + PD::BYTES + QD::lds_off(wave, s2), qoff[s2]);
    };
    constexpr int LPC = PD::NI + QD::NI;
    constexpr int DBKK = PD::KROWS;                   // tokens per chunk
    const int nkd = kend > kbeg ? (int)((kend - kbeg + DBKK - 1) / DBKK) : 0;
#pragma unroll
    for (int c = 0; c < NSTG - 1; ++c)
      if (c < nkd) issue(kbeg + (int64_t)c * DBKK, smem + c * DSTAGE);
    for (int kc = 0; kc < nkd; ++kc) {
      ring_barrier<LPC, NSTG>(nkd - 1 - kc);
      if (kc + NSTG - 1 < nkd) issue(kbeg + (int64_t)(kc + NSTG - 1) * DBKK, smem + ((kc + NSTG - 1) % NSTG) * DSTAGE);
      const char* buf = smem + (kc % NSTG) * DSTAGE;
      mfma_chunk<T, PD, QD, NS, MS, DKB / 32, true>(acc, buf + PD::BYTES, buf, qrow, prow, lane);
    }
  } else {
  auto load = [&](int64_t kc, PO& po, QO& qo) {
    const int kvalid = (int)((kend - kc) < BK ? (kend - kc) : BK);
    po.load_kmajor(Pb + kc * pld, pld, kvalid, tid);
    qo.load_kmajor(Qb + kc * qld, qld, kvalid, tid);
  };
  auto stage = [&](char* buf, const PO& po, const QO& qo) {
    po.stage_kmajor(buf, tid);
    qo.stage_kmajor(buf + PO::BYTES, tid);
  };

  if (nk > 0) {
    PO po;
    QO qo;
    load(kbeg, po, qo);
    stage(smem, po, qo);
    __syncthreads();
    for (int kc = 0; kc < nk; ++kc) {
      const bool more = kc + 1 < nk;
      if (more) load(kbeg + (int64_t)(kc + 1) * BK, po, qo);
      const char* buf = smem + (kc & 1) * STAGE;
      mfma_chunk<T, PO, QO, NS, MS>(acc, buf + PO::BYTES, buf, qrow, prow, lane);
      if (more) stage(smem + ((kc + 1) & 1) * STAGE, po, qo);
      __syncthreads();
    }
  }
  }  // main loops

  // out[m][n] at C + g*cgs + sp*css + (n/sub)*(M*sub) + m*sub + n%sub
  constexpr bool PERM = (ES == 2) || MX;
  constexpr int RUN = PERM ? 8 : 4, NRUN = 16 / RUN, RSTEP = PERM ? 16 : 8;
  const int h = lane >> 5;
#pragma unroll
  for (int ms = 0; ms < MS; ++ms) {
    const int64_t m = m0 + prow[ms] + (lane & 31);
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) {
#pragma unroll
      for (int t = 0; t < NRUN; ++t) {
        const int n = n0 + qrow[ns] + RSTEP * t + RUN * h;
        const int blk = n / a.sub;
        const int64_t off = (int64_t)g * a.c_group_stride + (int64_t)sp * a.c_split_stride +
                            ((int64_t)blk * a.M + m) * a.sub + (n - blk * a.sub);
        float v[RUN];
#pragma unroll
        for (int i = 0; i < RUN; ++i) v[i] = acc[ns][ms][RUN * t + i];
        if constexpr (OUT_F32) store_run<float, RUN>(static_cast<float*>(a.C) + off, v);
        else store_run<TO, RUN>(static_cast<TO*>(a.C) + off, v);
      }
    }
  }
}

// Dynamic LDS of one kernel: the 4-stage ring (16-bit) or two stages of the
// larger operand pair (f32), plus the schedule scratch of the row GEMMs.
template <typename T, int BM, int BN, bool WGRAD, bool PP = false>
constexpr size_t smem_for() {
  if constexpr (sizeof(T) == 2) {
    using C = TileCfg<BM, BN, WGRAD, PP>;
    return (size_t)C::NSTG * (BM + BN) * C::DKB + 64;   // direct-load ring
  } else {
    constexpr int nn = Operand<T, BM, false>::BYTES + Operand<T, BN, false>::BYTES;
    constexpr int nt = Operand<T, BM, false>::BYTES + Operand<T, BN, true>::BYTES;
    constexpr int tt = Operand<T, BM, true>::BYTES + Operand<T, BN, true>::BYTES;
    constexpr int m1 = nn > nt ? nn : nt;
    constexpr int m2 = m1 > tt ? m1 : tt;
    return 2 * (size_t)m2 + 64;
  }
}

}  // namespace

// ------------------------------------------------------- named kernels ------
// One plainly named kernel per (operation, dtype, tile) so profiles read well.

#define MOE_ROW_KERNEL(NAME, T, BM, BN, OP, EPI)                                                    \
  extern "C" __global__ void __launch_bounds__((TileCfg<BM, BN, false>::THREADS))                   \
      __attribute__((amdgpu_waves_per_eu(TileCfg<BM, BN, false>::WAVES_PER_EU))) NAME(RowGemmArgs a) {  \
    extern __shared__ __attribute__((aligned(16))) char smem[];                                   \
    row_gemm_body<T, BM, BN, OP, EPI, TileCfg<BM, BN, false>::WM, TileCfg<BM, BN, false>::WN>(a, smem);    \
  }
#define MOE_WGRAD_KERNEL(NAME, T, BM, BN, F32)                                                      \
  extern "C" __global__ void __launch_bounds__((TileCfg<BM, BN, true>::THREADS)) NAME(WgradArgs a) {    \
    extern __shared__ __attribute__((aligned(16))) char smem[];                                   \
    wgrad_body<T, BM, BN, F32, TileCfg<BM, BN, true>::WM, TileCfg<BM, BN, true>::WN>(a, smem);             \
  }

#define MOE_KERNEL_SET(T, TN, BM, BN)                                                                      \
  MOE_ROW_KERNEL(moe_gemm_gate_up_swiglu_##TN##_##BM##x##BN, T, BM, BN, OP_GU_FWD, EPI_SWIGLU_FWD)         \
  MOE_ROW_KERNEL(moe_gemm_down_##TN##_##BM##x##BN, T, BM, BN, OP_DOWN_FWD, EPI_STORE)                      \
  MOE_ROW_KERNEL(moe_gemm_down_f32out_##TN##_##BM##x##BN, T, BM, BN, OP_DOWN_FWD, EPI_STORE_F32)           \
  MOE_ROW_KERNEL(moe_gemm_down_dgrad_swiglu_##TN##_##BM##x##BN, T, BM, BN, OP_DOWN_DGRAD, EPI_SWIGLU_BWD)  \
  MOE_ROW_KERNEL(moe_gemm_gate_up_dgrad_##TN##_##BM##x##BN, T, BM, BN, OP_GU_DGRAD, EPI_STORE)             \
  MOE_ROW_KERNEL(moe_gemm_gate_up_dgrad_f32out_##TN##_##BM##x##BN, T, BM, BN, OP_GU_DGRAD, EPI_STORE_F32)  \
  MOE_ROW_KERNEL(moe_gemm_router_dx_f32out_##TN##_##BM##x##BN, T, BM, BN, OP_ROUTER_DX, EPI_STORE_F32)     \
  MOE_WGRAD_KERNEL(moe_wgrad_down_##TN##_##BM##x##BN, T, BM, BN, 0)                                        \
  MOE_WGRAD_KERNEL(moe_wgrad_gate_up_##TN##_##BM##x##BN, T, BM, BN, 0)                                     \
  MOE_WGRAD_KERNEL(moe_wgrad_down_f32out_##TN##_##BM##x##BN, T, BM, BN, 1)                                 \
  MOE_WGRAD_KERNEL(moe_wgrad_gate_up_f32out_##TN##_##BM##x##BN, T, BM, BN, 1)                              \
  MOE_WGRAD_KERNEL(moe_wgrad_router_f32out_##TN##_##BM##x##BN, T, BM, BN, 1)

#define MOE_ROW_KERNEL_SET(T, TN, BM, BN)                                                                  \
  MOE_ROW_KERNEL(moe_gemm_gate_up_swiglu_##TN##_##BM##x##BN, T, BM, BN, OP_GU_FWD, EPI_SWIGLU_FWD)         \
  MOE_ROW_KERNEL(moe_gemm_down_##TN##_##BM##x##BN, T, BM, BN, OP_DOWN_FWD, EPI_STORE)                      \
  MOE_ROW_KERNEL(moe_gemm_down_f32out_##TN##_##BM##x##BN, T, BM, BN, OP_DOWN_FWD, EPI_STORE_F32)           \
  MOE_ROW_KERNEL(moe_gemm_down_dgrad_swiglu_##TN##_##BM##x##BN, T, BM, BN, OP_DOWN_DGRAD, EPI_SWIGLU_BWD)  \
  MOE_ROW_KERNEL(moe_gemm_gate_up_dgrad_##TN##_##BM##x##BN, T, BM, BN, OP_GU_DGRAD, EPI_STORE)             \
  MOE_ROW_KERNEL(moe_gemm_gate_up_dgrad_f32out_##TN##_##BM##x##BN, T, BM, BN, OP_GU_DGRAD, EPI_STORE_F32)  \
  MOE_ROW_KERNEL(moe_gemm_router_dx_f32out_##TN##_##BM##x##BN, T, BM, BN, OP_ROUTER_DX, EPI_STORE_F32)

// 256 x 256 ping-pong row GEMMs (8 waves, two per SIMD)
#define MOE_ROW_KERNEL_PP(NAME, T, OP, EPI)                                                         \
  extern "C" __global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))          \
      NAME(RowGemmArgs a) {                                                                          \
    extern __shared__ __attribute__((aligned(16))) char smem[];                                     \
    row_gemm_body<T, 256, 256, OP, EPI, 2, 4, false, true>(a, smem);                                \
  }
#define MOE_WGRAD_KERNEL_PP(NAME, T, F32)                                                           \
  extern "C" __global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))          \
      NAME(WgradArgs a) {                                                                            \
    extern __shared__ __attribute__((aligned(16))) char smem[];                                     \
    wgrad_body<T, 256, 256, F32, 2, 4, false, true>(a, smem);                                       \
  }
#define MOE_ROW_KERNEL_SET_PP(T, TN)                                                                       \
  MOE_ROW_KERNEL_PP(moe_gemm_gate_up_swiglu_##TN##_256x256pp, T, OP_GU_FWD, EPI_SWIGLU_FWD)                \
  MOE_ROW_KERNEL_PP(moe_gemm_down_##TN##_256x256pp, T, OP_DOWN_FWD, EPI_STORE)                             \
  MOE_ROW_KERNEL_PP(moe_gemm_down_f32out_##TN##_256x256pp, T, OP_DOWN_FWD, EPI_STORE_F32)                  \
  MOE_ROW_KERNEL_PP(moe_gemm_down_dgrad_swiglu_##TN##_256x256pp, T, OP_DOWN_DGRAD, EPI_SWIGLU_BWD)         \
  MOE_ROW_KERNEL_PP(moe_gemm_gate_up_dgrad_##TN##_256x256pp, T, OP_GU_DGRAD, EPI_STORE)                    \
  MOE_ROW_KERNEL_PP(moe_gemm_gate_up_dgrad_f32out_##TN##_256x256pp, T, OP_GU_DGRAD, EPI_STORE_F32)         \
  MOE_ROW_KERNEL_PP(moe_gemm_router_dx_f32out_##TN##_256x256pp, T, OP_ROUTER_DX, EPI_STORE_F32)         \
  MOE_WGRAD_KERNEL_PP(moe_wgrad_down_##TN##_256x256pp, T, 0)                                               \
  MOE_WGRAD_KERNEL_PP(moe_wgrad_gate_up_##TN##_256x256pp, T, 0)                                            \
  MOE_WGRAD_KERNEL_PP(moe_wgrad_down_f32out_##TN##_256x256pp, T, 1)                                        \
  MOE_WGRAD_KERNEL_PP(moe_wgrad_gate_up_f32out_##TN##_256x256pp, T, 1)                                     \
  MOE_WGRAD_KERNEL_PP(moe_wgrad_router_f32out_##TN##_256x256pp, T, 1)

// the down dgrad with the rounding remainders (bf16 plans with few rows per expert)
#define MOE_DGRAD_LO_KERNEL(BM, BN)                                                                 \
  extern "C" __global__ void __launch_bounds__((TileCfg<BM, BN, false>::THREADS))                   \
      __attribute__((amdgpu_waves_per_eu(TileCfg<BM, BN, false>::WAVES_PER_EU)))                    \
      moe_gemm_down_dgrad_swiglu_lo_bf16_##BM##x##BN(RowGemmArgs a) {                                \
    extern __shared__ __attribute__((aligned(16))) char smem[];                                   \
    row_gemm_body<__bf16, BM, BN, OP_DOWN_DGRAD, EPI_SWIGLU_BWD, TileCfg<BM, BN, false>::WM,        \
                  TileCfg<BM, BN, false>::WN, false, false, true>(a, smem);                         \
  }
MOE_DGRAD_LO_KERNEL(128, 128)
MOE_DGRAD_LO_KERNEL(128, 256)
MOE_DGRAD_LO_KERNEL(256, 256)
extern "C" __global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
    moe_gemm_down_dgrad_swiglu_lo_bf16_256x256pp(RowGemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  row_gemm_body<__bf16, 256, 256, OP_DOWN_DGRAD, EPI_SWIGLU_BWD, 2, 4, false, true, true>(a, smem);
}

MOE_KERNEL_SET(__bf16, bf16, 256, 256)
MOE_ROW_KERNEL_SET_PP(__bf16, bf16)
MOE_ROW_KERNEL_SET_PP(_Float16, f16)
MOE_KERNEL_SET(__bf16, bf16, 128, 128)
MOE_ROW_KERNEL_SET(__bf16, bf16, 128, 256)
MOE_KERNEL_SET(_Float16, f16, 256, 256)
MOE_KERNEL_SET(_Float16, f16, 128, 128)
MOE_ROW_KERNEL_SET(_Float16, f16, 128, 256)
MOE_KERNEL_SET(float, f32, 128, 128)

// MX-fp8 expert GEMMs (128 x 128 tiles, 4 waves, 2-stage ring of 128-byte chunks)
#define MOE_MX_ROW_KERNEL(NAME, OP, EPI)                                                              \
  extern "C" __global__ void __launch_bounds__(256) NAME(RowGemmArgs a) {                          \
    extern __shared__ __attribute__((aligned(16))) char smem[];                                   \
    row_gemm_body<uint8_t, 128, 128, OP, EPI, 2, 2, true>(a, smem);                               \
  }
#define MOE_MX_WGRAD_KERNEL(NAME, F32)                                                                \
  extern "C" __global__ void __launch_bounds__(256) NAME(WgradArgs a) {                            \
    extern __shared__ __attribute__((aligned(16))) char smem[];                                   \
    wgrad_body<uint8_t, 128, 128, F32, 2, 2, true>(a, smem);                                      \
  }
MOE_MX_ROW_KERNEL(moe_mx_gemm_gate_up_swiglu_128x128, OP_GU_FWD, EPI_SWIGLU_FWD)
MOE_MX_ROW_KERNEL(moe_mx_gemm_down_128x128, OP_DOWN_FWD, EPI_STORE)
MOE_MX_ROW_KERNEL(moe_mx_gemm_down_f32out_128x128, OP_DOWN_FWD, EPI_STORE_F32)
MOE_MX_ROW_KERNEL(moe_mx_gemm_down_dgrad_swiglu_128x128, OP_DOWN_DGRAD, EPI_SWIGLU_BWD)
MOE_MX_ROW_KERNEL(moe_mx_gemm_gate_up_dgrad_128x128, OP_GU_DGRAD, EPI_STORE)
// 256 x 256 tiles, 8 waves (2 x 4), the same 2-stage ring of 128-byte chunks
// (one workgroup per CU); not for the SwiGLU backward, whose epilogue writes
// the token-axis codes block by block of a 128-row tile
#define MOE_MX_ROW_KERNEL_256(NAME, OP, EPI)                                                          \
  extern "C" __global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) NAME(RowGemmArgs a) { \
    extern __shared__ __attribute__((aligned(16))) char smem[];                                   \
    row_gemm_body<uint8_t, 256, 256, OP, EPI, 2, 4, true>(a, smem);                               \
  }
MOE_MX_ROW_KERNEL_256(moe_mx_gemm_gate_up_swiglu_256x256, OP_GU_FWD, EPI_SWIGLU_FWD)
MOE_MX_ROW_KERNEL_256(moe_mx_gemm_down_256x256, OP_DOWN_FWD, EPI_STORE)
MOE_MX_ROW_KERNEL_256(moe_mx_gemm_down_f32out_256x256, OP_DOWN_FWD, EPI_STORE_F32)
MOE_MX_ROW_KERNEL_256(moe_mx_gemm_gate_up_dgrad_256x256, OP_GU_DGRAD, EPI_STORE)
#define MOE_MX_WGRAD_KERNEL_256(NAME, F32)                                                            \
  extern "C" __global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) NAME(WgradArgs a) { \
    extern __shared__ __attribute__((aligned(16))) char smem[];                                   \
    wgrad_body<uint8_t, 256, 256, F32, 2, 4, true>(a, smem);                                      \
  }
MOE_MX_WGRAD_KERNEL_256(moe_mx_wgrad_down_256x256, 0)
MOE_MX_WGRAD_KERNEL_256(moe_mx_wgrad_gate_up_256x256, 0)
MOE_MX_WGRAD_KERNEL_256(moe_mx_wgrad_down_f32out_256x256, 1)
MOE_MX_WGRAD_KERNEL_256(moe_mx_wgrad_gate_up_f32out_256x256, 1)
MOE_MX_WGRAD_KERNEL(moe_mx_wgrad_down_128x128, 0)
MOE_MX_WGRAD_KERNEL(moe_mx_wgrad_gate_up_128x128, 0)
MOE_MX_WGRAD_KERNEL(moe_mx_wgrad_down_f32out_128x128, 1)
MOE_MX_WGRAD_KERNEL(moe_mx_wgrad_gate_up_f32out_128x128, 1)

namespace {

typedef void (*RowKernel)(RowGemmArgs);
typedef void (*WgradKernel)(WgradArgs);

struct KernelSet {
  RowKernel gu, down, down_f32, down_dgrad, gu_dgrad, gu_dgrad_f32, router_dx_f32;
  WgradKernel wgrad_down, wgrad_gate_up, wgrad_down_f32, wgrad_gate_up_f32, wgrad_router_f32;
  size_t lds_row, lds_wgrad;
  RowKernel down_dgrad_lo;   // bf16 only
};

#define MOE_KERNEL_TABLE(T, TN, BM, BN, LOK)                                                            \
  KernelSet{moe_gemm_gate_up_swiglu_##TN##_##BM##x##BN, moe_gemm_down_##TN##_##BM##x##BN,               \
            moe_gemm_down_f32out_##TN##_##BM##x##BN, moe_gemm_down_dgrad_swiglu_##TN##_##BM##x##BN,     \
            moe_gemm_gate_up_dgrad_##TN##_##BM##x##BN, moe_gemm_gate_up_dgrad_f32out_##TN##_##BM##x##BN,     \
            moe_gemm_router_dx_f32out_##TN##_##BM##x##BN,                                                   \
            moe_wgrad_down_##TN##_##BM##x##BN, moe_wgrad_gate_up_##TN##_##BM##x##BN,                      \
            moe_wgrad_down_f32out_##TN##_##BM##x##BN, moe_wgrad_gate_up_f32out_##TN##_##BM##x##BN,        \
            moe_wgrad_router_f32out_##TN##_##BM##x##BN, smem_for<T, BM, BN, false>(),                  \
            smem_for<T, BM, BN, true>(), LOK}

#define MOE_ROW_TABLE_PP(T, TN, LOK)                                                                    \
  KernelSet{moe_gemm_gate_up_swiglu_##TN##_256x256pp, moe_gemm_down_##TN##_256x256pp,                   \
            moe_gemm_down_f32out_##TN##_256x256pp, moe_gemm_down_dgrad_swiglu_##TN##_256x256pp,         \
            moe_gemm_gate_up_dgrad_##TN##_256x256pp, moe_gemm_gate_up_dgrad_f32out_##TN##_256x256pp,         \
            moe_gemm_router_dx_f32out_##TN##_256x256pp,                                                     \
            moe_wgrad_down_##TN##_256x256pp, moe_wgrad_gate_up_##TN##_256x256pp,                              \
            moe_wgrad_down_f32out_##TN##_256x256pp, moe_wgrad_gate_up_f32out_##TN##_256x256pp,                \
            moe_wgrad_router_f32out_##TN##_256x256pp, smem_for<T, 256, 256, false, true>(),                 \
            smem_for<T, 256, 256, true, true>(), LOK}

#define MOE_ROW_TABLE(T, TN, BM, BN, LOK)                                                               \
  KernelSet{moe_gemm_gate_up_swiglu_##TN##_##BM##x##BN, moe_gemm_down_##TN##_##BM##x##BN,               \
            moe_gemm_down_f32out_##TN##_##BM##x##BN, moe_gemm_down_dgrad_swiglu_##TN##_##BM##x##BN,     \
            moe_gemm_gate_up_dgrad_##TN##_##BM##x##BN, moe_gemm_gate_up_dgrad_f32out_##TN##_##BM##x##BN,     \
            moe_gemm_router_dx_f32out_##TN##_##BM##x##BN,                                                   \
            nullptr, nullptr, nullptr, nullptr, nullptr, smem_for<T, BM, BN, false>(), 0, LOK}

const KernelSet* kernel_set(int dt, int tile) {
  static const KernelSet bf16_256 = MOE_KERNEL_TABLE(__bf16, bf16, 256, 256, moe_gemm_down_dgrad_swiglu_lo_bf16_256x256);
  static const KernelSet bf16_128 = MOE_KERNEL_TABLE(__bf16, bf16, 128, 128, moe_gemm_down_dgrad_swiglu_lo_bf16_128x128);
  static const KernelSet bf16_128x256 =
      MOE_ROW_TABLE(__bf16, bf16, 128, 256, moe_gemm_down_dgrad_swiglu_lo_bf16_128x256);
  static const KernelSet f16_256 = MOE_KERNEL_TABLE(_Float16, f16, 256, 256, nullptr);
  static const KernelSet f16_128 = MOE_KERNEL_TABLE(_Float16, f16, 128, 128, nullptr);
  static const KernelSet f16_128x256 = MOE_ROW_TABLE(_Float16, f16, 128, 256, nullptr);
  static const KernelSet f32_128 = MOE_KERNEL_TABLE(float, f32, 128, 128, nullptr);
  static const KernelSet bf16_pp = MOE_ROW_TABLE_PP(__bf16, bf16, moe_gemm_down_dgrad_swiglu_lo_bf16_256x256pp);
  static const KernelSet f16_pp = MOE_ROW_TABLE_PP(_Float16, f16, nullptr);
  if (tile == TILE_256PP) return dt == DT_BF16 ? &bf16_pp : (dt == DT_F16 ? &f16_pp : nullptr);
  if (dt == DT_BF16) return tile == TILE_256 ? &bf16_256 : (tile == TILE_128x256 ? &bf16_128x256 : &bf16_128);
  if (dt == DT_F16) return tile == TILE_256 ? &f16_256 : (tile == TILE_128x256 ? &f16_128x256 : &f16_128);
  if (dt == DT_F32 && tile == 128) return &f32_128;
  if (dt == DT_MXFP8 && tile == 128) {
    constexpr size_t mx_lds = 2 * (128 + 128) * MX_DKB + 2 * (128 + 128) * 4 + 64;
    static const KernelSet mx_128{moe_mx_gemm_gate_up_swiglu_128x128, moe_mx_gemm_down_128x128,
                                  moe_mx_gemm_down_f32out_128x128, moe_mx_gemm_down_dgrad_swiglu_128x128,
                                  moe_mx_gemm_gate_up_dgrad_128x128, nullptr, nullptr,
                                  moe_mx_wgrad_down_128x128, moe_mx_wgrad_gate_up_128x128,
                                  moe_mx_wgrad_down_f32out_128x128, moe_mx_wgrad_gate_up_f32out_128x128,
                                  nullptr, mx_lds, mx_lds, nullptr};
    return &mx_128;
  }
  if (dt == DT_MXFP8 && tile == TILE_256) {
    constexpr size_t mx_lds = 2 * (256 + 256) * MX_DKB + 2 * (256 + 256) * 4 + 64;
    static const KernelSet mx_256{moe_mx_gemm_gate_up_swiglu_256x256, moe_mx_gemm_down_256x256,
                                  moe_mx_gemm_down_f32out_256x256, nullptr, moe_mx_gemm_gate_up_dgrad_256x256,
                                  nullptr, nullptr,
                                  moe_mx_wgrad_down_256x256, moe_mx_wgrad_gate_up_256x256,
                                  moe_mx_wgrad_down_f32out_256x256, moe_mx_wgrad_gate_up_f32out_256x256,
                                  nullptr, mx_lds, mx_lds, nullptr};
    return &mx_256;
  }
  return nullptr;
}

// More than 64 KB of dynamic LDS needs a per-kernel opt-in, done once per kernel.
hipError_t prepare(const void* k, size_t lds) {
  static std::mutex mu;
  static std::set<const void*> done;
  std::lock_guard<std::mutex> lk(mu);
  if (done.count(k)) return hipSuccess;
  hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e == hipSuccess) done.insert(k);
  return e;
}

}  // namespace

hipError_t launch_row_gemm(int dt, int op, int epi, int tile, const RowGemmArgs& a, hipStream_t s) {
  const KernelSet* set = kernel_set(dt, tile);
  if (!set) return hipErrorInvalidValue;
  RowKernel k = nullptr;
  switch (op) {
    case OP_GU_FWD: k = set->gu; break;
    case OP_DOWN_FWD: k = (epi == EPI_STORE_F32) ? set->down_f32 : set->down; break;
    case OP_DOWN_DGRAD: k = a.C_lo ? set->down_dgrad_lo : set->down_dgrad; break;
    case OP_GU_DGRAD: k = (epi == EPI_STORE_F32) ? set->gu_dgrad_f32 : set->gu_dgrad; break;
    case OP_ROUTER_DX: k = set->router_dx_f32; break;
    default: return hipErrorInvalidValue;
  }
  if (!k) return hipErrorInvalidValue;
  // every call writes C, except the MX SwiGLU backward, whose [dG | dU] codes are its product;
  // the SwiGLU forward writes H (C2), except with MX when both its codes are written
  if (!a.C && !(dt == DT_MXFP8 && op == OP_DOWN_DGRAD && a.Hq && a.Tq)) return hipErrorInvalidValue;
  if (op == OP_GU_FWD && !a.C2 && !(dt == DT_MXFP8 && a.Hq && a.Tq)) return hipErrorInvalidValue;
  if (a.C_lo && (op != OP_DOWN_DGRAD || !a.C2 || !a.C2_lo)) return hipErrorInvalidValue;
  // the f16 and MX-fp8 down dgrads write no w H rows
  if (op == OP_DOWN_DGRAD && a.C2 && (dt == DT_F16 || dt == DT_MXFP8)) return hipErrorInvalidValue;
  if (dt == DT_MXFP8 && (a.ldp % 128 || a.ldq % 128 || a.q_group_stride % 32 || !a.Ps || !a.Qs))
    return hipErrorInvalidValue;
  // token-axis codes of [dG | dU] (MX SwiGLU backward) or H (MX SwiGLU
  // forward), rows of ldt bytes (a multiple of 128)
  if (a.Tq && (dt != DT_MXFP8 || !((op == OP_DOWN_DGRAD && epi == EPI_SWIGLU_BWD) ||
                                   (op == OP_GU_FWD && epi == EPI_SWIGLU_FWD)) ||
               !a.Ts || a.ldt <= 0 || a.ldt % 128 || (a.offsets && !a.tpad)))
    return hipErrorInvalidValue;
  if (dt == DT_F32 && tile != TILE_128) return hipErrorInvalidValue;
  const int bm = tile_rows(tile), bn = tile_cols(tile);
  const int tile_n = (op == OP_GU_FWD) ? bn / 2 : bn;
  if (a.N % tile_n || a.K % (KB / dtype_bytes(dt))) return hipErrorInvalidValue;
  const int64_t n_ntiles = a.N / tile_n;
  int64_t mtiles;
  if (a.offsets) mtiles = (a.M + (int64_t)a.G * (bm - 1)) / bm;   // >= sum_g ceil(len_g / bm)
  else mtiles = (a.M + bm - 1) / bm;
  int64_t grid = mtiles * n_ntiles;
  grid = (grid + 7) / 8 * 8;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipError_t e = prepare((const void*)k, set->lds_row);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3((tile == TILE_256 || tile == TILE_256PP) ? 512 : 256),
                     set->lds_row, s, a);
  return hipGetLastError();
}

hipError_t launch_wgrad(int dt, int op, int tile, const WgradArgs& a, hipStream_t s) {
  const KernelSet* set = kernel_set(dt, tile);
  if (!set) return hipErrorInvalidValue;
  WgradKernel k = nullptr;
  switch (op) {
    case WG_DOWN: k = a.out_f32 ? set->wgrad_down_f32 : set->wgrad_down; break;
    case WG_GATE_UP: k = a.out_f32 ? set->wgrad_gate_up_f32 : set->wgrad_gate_up; break;
    case WG_ROUTER: k = set->wgrad_router_f32; break;
    default: return hipErrorInvalidValue;
  }
  if (!k || (op == WG_ROUTER && !a.out_f32) || (tile != TILE_128 && tile != TILE_256 && tile != TILE_256PP))
    return hipErrorInvalidValue;
  if (dt == DT_MXFP8 && (a.ldp % 128 || a.ldq % 128 || !a.offsets || !a.Ps || !a.Qs)) return hipErrorInvalidValue;
  const int bt = tile_rows(tile);                     // square tiles: 128 or 256
  if (a.M % bt || a.N % bt) return hipErrorInvalidValue;
  const int64_t chunk8 = 8 * (int64_t)(a.N / bt);     // whole rounds of XCD chunks (xcd_chunked)
  int64_t grid = (int64_t)a.G * a.splits * (a.M / bt) * (a.N / bt);
  grid = (grid + chunk8 - 1) / chunk8 * chunk8;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipError_t e = prepare((const void*)k, set->lds_wgrad);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(tile == TILE_128 ? 256 : 512),
                     set->lds_wgrad, s, a);
  return hipGetLastError();
}

}  // namespace moe
