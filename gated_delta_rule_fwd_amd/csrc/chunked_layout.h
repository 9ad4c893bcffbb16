// Memory plans of the two chunked kernels, shared by the kernels and the host
// launcher (which sizes the dynamic LDS and the workspace and rejects shapes
// that do not fit).
//
//   prep kernel   one workgroup per (sequence, head, chunk): everything that
//                 does not depend on the state, written to a per-chunk record
//   state kernel  one workgroup per (sequence, head, value slice): walks the
//                 chunks in order, reads the records, keeps the state
#pragma once

#include <stddef.h>

namespace kda {

constexpr size_t kMaxLds = 160 * 1024;

namespace chunked_layout {
constexpr size_t mx(size_t a, size_t b) { return a > b ? a : b; }
constexpr size_t al(size_t a) { return (a + 255) & ~size_t(255); }
}  // namespace chunked_layout

// Per-chunk record in the workspace (global memory), all tiles row-major with
// one row per token of the chunk.  OpBytes: 2 (fp16 operands) or 4 (fp32).
//   Q    q normalised and scaled; per-channel decay: times exp(G)
//   K    k normalised; per-channel decay: times exp(Gx)
//   F    per-channel decay only: k normalised times exp(G_last - G)
//   Tu   T diag(beta), T = (I + A)^-1, zero above the block diagonal  [C][C]
//   P    masked decayed q k^T, zero above the block diagonal          [C][C]
//   vec  fp32: exp(G), exp(Gx), exp(G_last - G) (each C), misc[16] with
//        misc[0] = exp(G_last); per-channel: exp(G_last) per key channel [DK]
template <int DK, int C, int OpBytes, bool Chan>
struct RecLayout {
  static constexpr size_t kTile = size_t(C) * DK * OpBytes;
  static constexpr size_t kCC = size_t(C) * C * OpBytes;
  static constexpr int kTiles = Chan ? 3 : 2;       // Q, K (, F)
  static constexpr size_t oQ = 0;
  static constexpr size_t oK = oQ + kTile;
  static constexpr size_t oF = oK + kTile;
  static constexpr size_t oTu = oQ + kTiles * kTile;
  static constexpr size_t oP = oTu + kCC;
  static constexpr size_t oVec = oP + kCC;
  static constexpr int vEG = 0, vEGx = C, vEF = 2 * C, vMisc = 3 * C, vDecC = 3 * C + 16;
  static constexpr int kVecFloats = 3 * C + 16 + (Chan ? DK : 0);
  static constexpr size_t bytes = chunked_layout::al(oVec + size_t(kVecFloats) * 4);
};

// LDS of the prep kernel.
template <int DK, int C, int OpBytes>
struct PrepLayout {
  static constexpr int NB = C / 16;                 // 16-token blocks per chunk
  static constexpr int NCOL = C < 32 ? 32 : C;      // token columns read by 32-wide k steps
  static constexpr int PAD = 16 / OpBytes;          // 16-byte row padding
  static constexpr int LDK = DK + PAD;              // row stride of [C][DK] operand tiles
  static constexpr int LC = NCOL + PAD;             // row stride of the [C][tokens] P tile
  static constexpr int LF = C + 4;                  // row stride of fp32 [C][C] tiles
  static constexpr int KinvBytes = OpBytes == 2 ? 2 : 4;

  static constexpr size_t kRowTile = size_t(C) * LDK * OpBytes;     // [C][DK]
  static constexpr size_t kCC = size_t(C) * LC * OpBytes;            // [C][tokens] operand
  static constexpr size_t kF32CC = size_t(C) * LF * 4;               // [C][C] fp32
  static constexpr size_t kGst = size_t(C) * DK * OpBytes;           // staged per-channel gate

  // Regions and what they hold:
  //   Q    q normalised (per-channel: and decayed)                load .. Gram
  //   K    k normalised (per-channel: and decayed)                load .. Gram
  //   P    masked decayed q k^T                                    Gram .. record
  //   AM   fp32 A (Gram .. inverse); per-channel: staged gate first (load)
  //   RA   per-channel Gram factors Kb, Kinv (load .. Gram)  |  fp32 T (inverse .. record)
  static constexpr size_t oQ = 0;
  static constexpr size_t oK = chunked_layout::al(oQ + kRowTile);
  static constexpr size_t oP = chunked_layout::al(oK + kRowTile);
  static constexpr size_t oAM = chunked_layout::al(oP + kCC);
  static constexpr size_t szAM(bool ch) { return ch ? chunked_layout::mx(kF32CC, kGst) : kF32CC; }
  static constexpr size_t oRA(bool ch) { return chunked_layout::al(oAM + szAM(ch)); }
  static constexpr size_t oKinv(bool ch) { return chunked_layout::al(oRA(ch) + kRowTile); }  // after Kb
  static constexpr size_t szRA(bool ch) {
    return chunked_layout::mx(ch ? (oKinv(ch) - oRA(ch)) + size_t(C) * LDK * KinvBytes : 0, kF32CC);
  }
  // D[i][j] (decay of the blocks strictly between j and i) is needed for i - j >= 2
  static constexpr int ND = NB >= 3 ? (NB - 2) * (NB - 1) / 2 : 1;
  static constexpr int dslot(int i, int j) { return (i - 2) * (i - 1) / 2 + j; }
  // fp32 vectors: bt Gi Ge (each C), misc[16]; per-channel: tau[NB] Cb[NB] rsq[NB] D[ND] (each DK)
  static constexpr int kVecRows = 3;
  static constexpr int kChanVecs = 3 * NB + ND;
  static constexpr size_t oVec(bool ch) { return chunked_layout::al(oRA(ch) + szRA(ch)); }
  static constexpr size_t szVec(bool ch) {
    return size_t(kVecRows) * C * 4 + 64 + (ch ? size_t(kChanVecs) * DK * 4 : 0);
  }
  static constexpr size_t bytes(bool ch) { return chunked_layout::al(oVec(ch) + szVec(ch)); }
};

// LDS of the state kernel: one chunk's record (padded rows) and its values.
template <int DK, int DVS, int C, int OpBytes, bool Chan>
struct StateLayout {
  static constexpr int NB = C / 16;
  static constexpr int NCOL = C < 32 ? 32 : C;
  static constexpr int PAD = 16 / OpBytes;
  static constexpr int LDK = DK + PAD;
  static constexpr int LDV = DVS + PAD;
  static constexpr int LC = NCOL + PAD;
  static constexpr size_t kRowTile = size_t(C) * LDK * OpBytes;
  static constexpr size_t kCC = size_t(C) * LC * OpBytes;
  static constexpr size_t oQ = 0;
  static constexpr size_t oK = chunked_layout::al(oQ + kRowTile);
  static constexpr size_t oF = chunked_layout::al(oK + kRowTile);
  static constexpr size_t oTu = chunked_layout::al(oF + (Chan ? kRowTile : 0));
  static constexpr size_t oP = chunked_layout::al(oTu + kCC);
  static constexpr size_t oV = chunked_layout::al(oP + kCC);
  static constexpr size_t oVec = chunked_layout::al(oV + size_t(C) * LDV * OpBytes);
  static constexpr int kVecFloats = RecLayout<DK, C, OpBytes, Chan>::kVecFloats;
  static constexpr size_t bytes = chunked_layout::al(oVec + size_t(kVecFloats) * 4);
};

}  // namespace kda
