/*
 * zs_offload_pieces.h -- internal interface between the host update
 * (offload_cpu.cpp) and the pipelined ZeRO-Offload step (zeroshard.hip):
 * the update of a partition whose gradient reaches host memory piece by
 * piece. Not part of the C ABI.
 */
#ifndef ZS_OFFLOAD_PIECES_H
#define ZS_OFFLOAD_PIECES_H

#include <stdint.h>

#include "zeroshard.h"

namespace zs_host {

/* Hooks of update_in_pieces. arrived(ctx, k) is called once per piece, by
 * the first thread that needs piece k, and returns 0 once that piece's
 * gradient is in host memory (anything else stops the update). updated(ctx,
 * k) is called once per updated piece, by the thread that finished the
 * piece's last part, as soon as its master, m, v and 16-bit parameters are
 * final. Both may be called from any pool thread. */
struct PieceHooks {
  void *ctx;
  int (*arrived)(void *ctx, int piece);
  void (*updated)(void *ctx, int piece);
};

/* The update of zs_cpu_update over [0, n), in pieces [cuts[k], cuts[k+1])
 * for k < pieces (cuts[0] = 0, cuts[pieces] = n, non-decreasing): every pool
 * thread takes its share of each piece in order, so the update of piece k
 * overlaps the arrival of the pieces after it. Returns ZS_OK, an argument
 * status as zs_cpu_update (and ZS_ERR_INVALID_ARG for bad cuts or hooks), or
 * ZS_ERR_HIP when arrived() reported a failure: then the pieces from the
 * failed one on are not updated, earlier ones are. n == 0 calls no hook. */
int update_in_pieces(float *master, float *m, float *v, const float *grad, uint64_t n,
                     const zs_adamw_hparams *hp, void *params16, int param_dtype, int threads,
                     const uint64_t *cuts, int pieces, const PieceHooks &hooks);

}  // namespace zs_host

#endif /* ZS_OFFLOAD_PIECES_H */
