// Direct-to-LDS staging for the bf16 attention backward: the dQ kernel's key tile images (K rows,
// V rows, K^T) and the dK/dV kernel's 32-query tile images. Built on the copy primitive and
// padded layouts of attn_fwd_lds.h.
#pragma once

#include "attn_fwd_lds.h"

namespace moc {

// Key tile images of the query-centric dQ kernel: for every 64 aligned keys of a (b, h), the
// bytes of one LDS stage part - K rows and V rows (64 rows each, pitch KROW chunks) and K^T
// (D rows of 64 keys, pitch VROW chunks) - padding included, rows past L zero. A stage holds the
// rows of tile j and the K^T of tile j-1, so staging it is two linear copies of 1 KB pieces
// whose only per-lane value is the lane's 16-byte offset.
template <int D>
struct KvImage {
  using LT = LdsTiles<D>;
  static constexpr int ROWBLK = 2 * LT::KBLK;          // 1 KB pieces of the K and V rows
  static constexpr int NBLK = ROWBLK + LT::VBLK;        // + the K^T piece
  static constexpr int BYTES = NBLK * 1024;             // one image = one stage
};

template <int D, int NW>
struct KvStageCopier {
  using KI = KvImage<D>;
  static constexpr int SLOTS = (KI::NBLK + NW - 1) / NW;
  int wv;
  uint32_t voff;

  __device__ __forceinline__ void init(int wave, int ln) {
    wv = wave;
    voff = static_cast<uint32_t>(ln) * 16u;
  }

  __device__ __forceinline__ int count() const { return KI::NBLK / NW + (wv < KI::NBLK % NW); }

  // rows of image `rows_img`, K^T of image `kt_img`, into the stage at LDS byte address lds
  __device__ __forceinline__ void issue(uint32_t lds, const char* rows_img,
                                        const char* kt_img) const {
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
      const int blk = wv + i * NW;
      if (blk >= KI::NBLK) break;
      copy16_to_lds((blk < KI::ROWBLK ? rows_img : kt_img) + blk * 1024, voff, lds + blk * 1024);
    }
  }
};

// ---------------------------------------------------------------------------------------------
// Query tiles of the key-centric backward: 32 consecutive (aligned) query positions of one
// (b, h), staged as Q rows and dO rows (pitch D/8 + 1 chunks, A operands of S = Q K^T and
// dP = dO V^T), Q^T and dO^T rows (D rows of 32 queries, pitch 5 chunks, B operands of
// dK += dS^T Q and dV += P^T dO), and one block holding lse2[32] and D[32]. The odd pitches keep
// the 16 lanes of an LDS read pass on 16 different bank slots. The tiles are built in global
// memory as this exact byte image (padding included), so staging one is a linear copy.
template <int D>
struct QTiles {
  static constexpr int T = 32;                          // queries per tile
  static constexpr int RROW = D / 8 + 1;                // row pitch (chunks)
  static constexpr int TROW = T / 8 + 1;                // transposed row pitch (chunks)
  static constexpr int RBLK = (T * RROW + 63) / 64;     // 1 KB blocks of one row tile
  static constexpr int TBLK = (D * TROW + 63) / 64;     // 1 KB blocks of one transposed tile
  static constexpr int NBLK = 2 * RBLK + 2 * TBLK + 1;
  static constexpr int BYTES = NBLK * 1024;
  static constexpr int Q_OFF = 0;
  static constexpr int DO_OFF = RBLK * 1024;
  static constexpr int QT_OFF = 2 * RBLK * 1024;
  static constexpr int DOT_OFF = (2 * RBLK + TBLK) * 1024;
  static constexpr int ST_OFF = (2 * RBLK + 2 * TBLK) * 1024;  // lse2[32] then D[32] (fp32)
};

// Direct-to-LDS copies of one wave (of NW) for one query tile image (QTiles layout): the
// wave copies the 1 KB pieces wv, wv + NW, ...; a lane moves bytes 16 lane .. 16 lane + 15 of
// each, so the only per-lane value is that one offset.
template <int D, int NW>
struct QTileCopier {
  using QT = QTiles<D>;
  static constexpr int SLOTS = (QT::NBLK + NW - 1) / NW;
  int wv;
  uint32_t voff;

  __device__ __forceinline__ void init(int wave, int ln) {
    wv = wave;
    voff = static_cast<uint32_t>(ln) * 16u;
  }

  __device__ __forceinline__ int count() const {
    return QT::NBLK / NW + (wv < QT::NBLK % NW);
  }

  __device__ __forceinline__ void issue(uint32_t lds, const char* img) const {
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
      const int blk = wv + i * NW;
      if (blk >= QT::NBLK) break;
      copy16_to_lds(img + blk * 1024, voff, lds + blk * 1024);
    }
  }
};

}  // namespace moc
