// Memory plans of the two chunked kernels, shared by the kernels and the host
// launcher (which sizes the dynamic LDS and the workspace and rejects shapes
// that do not fit).
//
//   prep kernel   one workgroup per (sequence, head, chunk): everything that
//                 does not depend on the state, written to a per-chunk record
//   state kernel  one workgroup per (sequence, head, value slice): walks the
//                 chunks in order, reads the records, keeps the state
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace kda {

constexpr size_t kMaxLds = 160 * 1024;

namespace chunked_layout {
constexpr size_t mx(size_t a, size_t b) { return a > b ? a : b; }
constexpr size_t al(size_t a) { return (a + 255) & ~size_t(255); }
}  // namespace chunked_layout

// XOR swizzle of the 16-byte pieces of a row of PPR pieces: the piece p of
// row r is stored at position p ^ swz<PPR>(r).  The LDS serves 128 bytes per
// step (32 banks): 8 lanes of a 16-byte read, 16 lanes of an 8-byte read.
// With the rows copied unpadded into LDS this swizzle makes (a) 16-byte reads
// of one piece column by 16 consecutive rows conflict-free and (b) the
// transposed 8-byte token reads (4 consecutive rows, 4 consecutive 8-byte
// pieces of a half) two-way, the least a fixed half allows.
template <int PPR>
__host__ __device__ constexpr int swz(int r) {
  return PPR >= 32 ? (r & 15)
       : PPR == 16 ? (((r & 1) << 2) | ((r >> 1) & 3) | (r & 8))
       : PPR == 8  ? (((r & 1) << 2) | ((r >> 1) & 3))
       : PPR == 4  ? ((r >> 1) & 3)
       : PPR == 2  ? ((r >> 2) & 1)
                   : 0;
}
// Byte offset of byte `b` of row r in a swizzled tile with PPR pieces per row.
template <int PPR>
__host__ __device__ constexpr int swz_off(int r, int b) {
  return r * PPR * 16 + (((b >> 4) ^ swz<PPR>(r)) << 4) + (b & 15);
}
// Value rows (activations, read only transposed: 4 consecutive rows x 16
// columns per 16 lanes): conflict-free with this swizzle.
template <int PPR>
__host__ __device__ constexpr int swzv(int r) {
  return PPR >= 8 ? 2 * (r & 3) : PPR == 4 ? 2 * ((r >> 1) & 1) : 0;
}
template <int PPR>
__host__ __device__ constexpr int swzv_off(int r, int b) {
  return r * PPR * 16 + (((b >> 4) ^ swzv<PPR>(r)) << 4) + (b & 15);
}
// Stored position of element e of a record row: within each 32-element group
// the 4-element subgroups are kept in the order 0 4 1 5 2 6 3 7, so the
// operand of an MFMA lane (elements 4g..4g+3 and 16+4g..16+4g+3 of a group)
// is 8 consecutive stored elements.
__host__ __device__ constexpr int perm_pos(int e) {
  return (e & ~31) + 4 * (2 * ((e >> 2) & 3) + ((e >> 4) & 1)) + (e & 3);
}

// Per-chunk record: the image of one chunk in the state kernel's LDS.  Each
// tile has one row per token of the chunk, rows unpadded and swizzled (swz
// above), elements in perm_pos order (raw rows below: natural order).
// OpBytes: 2 (fp16 operands) or 4 (fp32).
//   Q    q normalised and scaled; per-channel decay: times exp(G)
//   K    k normalised; per-channel decay: times exp(Gx)
//   F    per-channel decay only: k normalised times exp(G_last - G)
//   Tu   T diag(beta), T = (I + A)^-1, zero above the block diagonal  [C][NCOL]
//   P    masked decayed q k^T, zero above the block diagonal          [C][NCOL]
//        (NCOL = max(C, 32): the columns a 32-wide k step reads)
//   vec  fp32: exp(G), exp(Gx), exp(G_last - G) (each C), misc[16] with
//        misc[0] = exp(G_last); per-channel: exp(G_last) per key channel [DK];
//        raw rows: G and k's row factor fk (each C), and fk also folded
//        into exp(Gx) and exp(G_last - G)
// The workspace holds bytes [gOff, bytes) of the image per chunk.  Raw rows
// (bf16 activations, no per-channel decay, C >= 32): the image starts with q
// and k as they are (bf16, natural element order), which the state kernel
// copies from the inputs itself, and P is not stored: the state kernel forms
// it from those rows, the row factors and G.  The record is then Tu and the
// vectors only.
template <int DK, int C, int OpBytes, bool Chan>
struct RecLayout {
  static constexpr bool kRawK = !Chan && OpBytes == 2 && C >= 32;
  static constexpr int PPRK = DK * OpBytes / 16;   // pieces per Q/K/F row
  static constexpr int NCOL = C < 32 ? 32 : C;
  static constexpr int PPRC = NCOL * OpBytes / 16; // pieces per Tu/P row
  static constexpr size_t kTile = size_t(C) * DK * OpBytes;
  static constexpr size_t kCC = size_t(C) * NCOL * OpBytes;
  static constexpr int kTiles = Chan ? 3 : 2;       // Q, K (, F)
  static constexpr size_t oQ = kRawK ? kTile : 0;
  static constexpr size_t oK = kRawK ? 0 : kTile;
  static constexpr size_t oF = 2 * kTile;
  static constexpr size_t oTu = kTiles * kTile;
  static constexpr size_t oP = oTu + kCC;           // not with raw rows
  static constexpr size_t oVec = kRawK ? oTu + kCC : oP + kCC;
  static constexpr int vEG = 0, vEGx = C, vEF = 2 * C, vMisc = 3 * C, vDecC = 3 * C + 16;
  static constexpr int vG = 3 * C + 16, vFK = 4 * C + 16;   // raw rows
  static constexpr int kVecFloats = 3 * C + 16 + (Chan ? DK : 0) + (kRawK ? 2 * C : 0);
  static constexpr size_t bytes = chunked_layout::al(oVec + size_t(kVecFloats) * 4);
  static constexpr size_t gOff = kRawK ? 2 * kTile : 0;
  static constexpr size_t gBytes = bytes - gOff;
};

// LDS of the prep kernel; Raw: raw rows in the record (no q tile here).
template <int DK, int C, int OpBytes, bool Raw>
struct PrepLayout {
  static constexpr int NB = C / 16;                 // 16-token blocks per chunk
  static constexpr int NQ = C / 4;                  // 4-token quarters per chunk (per-channel decay)
  static constexpr int NCOL = C < 32 ? 32 : C;      // token columns read by 32-wide k steps
  static constexpr int PAD = 16 / OpBytes;          // 16-byte row padding
  static constexpr int LDK = DK + PAD;              // row stride of [C][DK] operand tiles
  static constexpr int LC = NCOL + PAD;             // row stride of the [C][tokens] P tile
  static constexpr int LF = C + 4;                  // row stride of fp32 [C][C] tiles

  static constexpr size_t kRowTile = size_t(C) * LDK * OpBytes;     // [C][DK]
  static constexpr size_t kCC = size_t(C) * LC * OpBytes;            // [C][tokens] operand
  static constexpr size_t kF32CC = size_t(C) * LF * 4;               // [C][C] fp32
  static constexpr size_t kGst = size_t(C) * DK * OpBytes;           // staged per-channel gate

  // Regions and what they hold:
  //   Q    q normalised; per-channel decay: times the decay products of its
  //        quarter (Gram of the diagonal blocks), then of its block (the
  //        off-diagonal ones)                                       load .. Gram
  //        (none with raw rows)
  //   K    k normalised; per-channel decay: likewise                load .. Gram
  //   AM   fp32 A (Gram .. inverse); per-channel: staged gate first (load)
  //   KB   per-channel decay: k decayed to the end of its quarter, then of
  //        its block                                                load .. Gram
  //   T    fp32 T: over the Q (per-channel) or the Q and K tiles (otherwise)
  //        where it fits, dead after the Gram; else a region of its own
  // (P goes from the MFMA accumulators straight to the record.)
  static constexpr size_t oQ = 0;
  static constexpr size_t oK = Raw ? 0 : chunked_layout::al(oQ + kRowTile);
  static constexpr size_t oAM = chunked_layout::al(oK + kRowTile);
  static constexpr size_t szAM(bool ch) { return ch ? chunked_layout::mx(kF32CC, kGst) : kF32CC; }
  static constexpr size_t oKB = chunked_layout::al(oAM + szAM(true));
  static constexpr bool kTinQK = kF32CC <= oAM - oQ;   // T fits over Q and K
  static constexpr bool kTinQ = kF32CC <= kRowTile;    // T fits over Q
  // the T region
  static constexpr size_t oRA(bool ch) {
    return ch ? (kTinQ ? oQ : chunked_layout::al(oKB + kRowTile))
              : (kTinQK ? oQ : chunked_layout::al(oAM + szAM(false)));
  }
  static constexpr size_t tilesEnd(bool ch) {
    return ch ? chunked_layout::al(chunked_layout::mx(oKB + kRowTile, oRA(true) + kF32CC))
              : (kTinQK ? chunked_layout::al(oAM + szAM(false)) : chunked_layout::al(oRA(false) + kF32CC));
  }
  // per-channel decay: off-diagonal block pairs (i, j) with i - j >= 2 take
  // the decay of the blocks strictly between them as a scale, D[ddslot]
  static constexpr int NDD = NB >= 3 ? (NB - 1) * (NB - 2) / 2 : 1;
  static constexpr int ddslot(int i, int j) { return (i - 2) * (i - 1) / 2 + j; }
  static constexpr int kWQ = 12;                    // within-quarter sums per quarter
  static constexpr int kWQD = NQ * kWQ > NDD * DK ? NQ * kWQ : NDD * DK;
  // fp32 vectors: bt Gi Ge qk (each C), misc[16]; per-channel: tau4[NQ][DK]
  // (the decay factor of each quarter), then the within-quarter sums [NQ][12],
  // later (same place) D[NDD][DK]; on the mild path the chunk's log decay
  // per channel, [DK]
  static constexpr int kVecRows = 4;
  static constexpr size_t oVec(bool ch) { return tilesEnd(ch); }
  static constexpr size_t szVec(bool ch) {
    return size_t(kVecRows) * C * 4 + 64 + (ch ? (size_t(NQ) * DK + kWQD) * 4 : 0);
  }
  static constexpr size_t bytes(bool ch) { return chunked_layout::al(oVec(ch) + szVec(ch)); }
};

// LDS of the state kernel: NBUF buffers, each one chunk's record image
// followed by its value rows ([C][DVS] activations, rows swizzled).  With two
// buffers the next chunk is copied in while the current one is computed.
//
// With raw rows (see RecLayout) the helper waves also form P for the
// owners: each forms some of its 16 x 16 blocks, into the fp16 operand
// fragments (PF, one 1 KiB fragment per 16-token row block and 32-token k
// step), and the row factors of q (FQ, one float per token), then sets its
// flag (ints after FQ) to the chunk + 1.
// Helper waves of the state kernel for a slice of DVS value columns: as many
// as the DVS / 16 owner waves, and at least two (so that a 16-column slice
// shares P and the copies between two waves).
template <int DVS> constexpr int state_helpers() { return DVS / 16 > 2 ? DVS / 16 : 2; }

template <int DK, int DVS, int C, int OpBytes, int ActBytes, bool Chan>
struct StateLayout {
  using R = RecLayout<DK, C, OpBytes, Chan>;
  static constexpr int PPRV = DVS * ActBytes / 16;   // pieces per value row
  // the record's bytes in the image, padded to whole 1 KiB copies for each of
  // the helper waves that issue them
  static constexpr size_t kRecSlot = size_t(1024) * state_helpers<DVS>();
  static constexpr size_t kRecLds = (R::gBytes + kRecSlot - 1) / kRecSlot * kRecSlot;
  static constexpr size_t oV = R::gOff + kRecLds;
  static constexpr size_t kBuf = chunked_layout::al(oV + size_t(C) * DVS * ActBytes);
  static constexpr size_t kTouch = R::kRawK ? 0 : 256;   // the prefetch slot (below)
  static constexpr int NBUF = 2 * kBuf + kTouch <= kMaxLds ? 2 : 1;
  static constexpr int NBT = C / 16;
  static constexpr int kNPF = NBT * (NBT + 2) / 4;   // P fragments: sum over row blocks ib of ib/2 + 1
  static constexpr bool kHelperP = R::kRawK && NBUF == 2;
  static constexpr size_t oPF = NBUF * kBuf;
  static constexpr size_t oFQ = oPF + size_t(kNPF) * 1024;
  static constexpr size_t oFlags = oFQ + chunked_layout::al(size_t(C) * 4);
  static constexpr size_t kFlags = 256;
  // the 256-byte landing slot of the L2 prefetch loads (never read; none
  // with raw rows, which are not prefetched)
  static constexpr size_t oTouch = kHelperP ? oFlags + kFlags : NBUF * kBuf;
  // raw rows need the helper-formed P: otherwise no plan (more than the LDS)
  static constexpr size_t bytes = R::kRawK && !kHelperP ? kMaxLds + 1 : oTouch + kTouch;
};

}  // namespace kda
