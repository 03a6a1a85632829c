/*
 * tfl_audit.h -- one extra entry point exported only by the audit build of
 * the library (libtfl_audit.so, compiled with TFL_AUDIT=1), which the tests
 * load beside the product library libtfl.so.
 *
 * The audit build checks two statements of "KernelForge", "Challenges"
 * about a causal attention loop:
 *  - evaluating the mask only on the key tiles that straddle the diagonal
 *    (here also the padding boundary) is bit-identical to evaluating it on
 *    every tile: every attention kernel of the audit build masks every tile
 *    it visits, and its outputs must equal the product build's bit for bit;
 *  - a causal loop visits only the key tiles that hold an allowed key, which
 *    at full length is M(M+1)/2 of M^2 tiles (the floor (M+1)/2M): the audit
 *    build adds the tiles its attention kernels visit to device counters.
 * Apart from that, the audit build runs the same kernels as the product.
 */
#ifndef TFL_AUDIT_H
#define TFL_AUDIT_H

#include "tfl.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Counter slots (uint64 each, 8 slots): key tiles staged per workgroup and
 * scored per 16-query wave by the layer-wise attention kernels (slots 0, 1),
 * 32-key chunks scored per 16-query wave by the fused SEQ kernel (slot 2),
 * key tiles staged per task and scored per wave by the PQ attention tasks
 * (slots 3, 4), and the layer-wise attention workgroups and PQ attention
 * tasks that took the hi/lo split scores (slot 5) or reference-free bounded
 * weights (slot 6).  The
 * small fused kernel scores key by key (no tiles) and adds nothing. */
enum { TFL_AUDIT_SLOTS = 8 };

/* counters: device memory of TFL_AUDIT_SLOTS uint64 values, 8-byte aligned,
 * owned by the caller, which zeroes it; every later tfl_forward in the
 * process adds to it with device atomics.  NULL detaches.  Process-wide, not
 * thread-safe. */
tfl_status tfl_audit_attach(void *counters);

#ifdef __cplusplus
}
#endif

#endif /* TFL_AUDIT_H */
