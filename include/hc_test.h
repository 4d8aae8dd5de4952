/*
 * hc_test.h — hooks of the test build of the library (libhc_test.so, the same
 * sources compiled with HC_TEST_HOOKS).  The product library libhc.so does not
 * export hc_test_hook.  The tests use them to drive the failure paths of the
 * C ABI (include/hc.h) from the host, keeping every kernel's indexes in range:
 * a HIP launch failure (HC_E_HIP, then HC_E_STATE), a kernel that finds an
 * inconsistent device state (HC_E_DEVICE, then HC_E_STATE), a pinned host
 * allocation that fails inside hc_create (which must leave nothing allocated:
 * the page "Making KV offload correct", section "A grouped allocation is a
 * transaction"), and victim slots poisoned before their fill (the page "From
 * 1M Total to 15+ × 1M Contexts: GLM-5.3 KV Cache Offloading", section "GPU
 * cache management has hazards too": a slot filled in a round must not be read
 * by another block of that round).
 */
#ifndef HC_TEST_H
#define HC_TEST_H

#include <stdint.h>

#include "hc.h"

#ifdef __cplusplus
extern "C" {
#endif

#define HC_TEST_FAIL_LAUNCH   1  /* ctx: the next hc_step fails as if its first launch had
                                    failed; nothing of it is enqueued                  */
#define HC_TEST_FORCE_SELECT  2  /* ctx: the next hc_step's select kernels report an
                                    inconsistent scan state (and keep every index in
                                    range: the gather then reads slot 0)               */
#define HC_TEST_CORRUPT_LRU   3  /* ctx: waits for the context, then marks every slot of
                                    every unit used with an empty LRU queue, so the
                                    next step that misses finds no victim              */
#define HC_TEST_FAIL_PINNED   4  /* NULL ctx: grant `arg` more pinned host allocations,
                                    then fail one (arg < 0: never fail)                */
#define HC_TEST_PINNED_BYTES  5  /* NULL ctx: *out = pinned host bytes the library holds */
#define HC_TEST_POISON_VICTIMS 6 /* ctx: arg != 0: before each gather, a sentinel over every
                                    victim slot (a read of a slot before its fill would
                                    reach the output); arg = 0: off                   */

hc_status hc_test_hook(hc_ctx* ctx, int kind, int64_t arg, uint64_t* out);

#ifdef __cplusplus
}
#endif
#endif /* HC_TEST_H */
