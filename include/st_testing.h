/*
 * st_testing.h -- test-only controls of libst.so's launch planners.
 *
 * Not for production callers.  Every planner in the library chooses kernel
 * shapes, split sizes and workspace sizes from the call's arguments alone.
 * A test suite that wants to drive each kernel shape and each split path on
 * small inputs installs an override here; a process that never calls
 * st_testing_set_plan gets the planners' own choices, always.
 */
#ifndef ST_TESTING_H
#define ST_TESTING_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t attn_shape;      /* -1: planner's choice; 0..6: the streaming attention kernel's
                              shape (row groups, row blocks) = (1,1) (1,2) (1,4) (2,4) (4,4)
                              (2,2) (4,2)                                                  */
  int32_t attn_target_wg;  /* 0: planner's choice; > 0: workgroups the split count aims for */
  int32_t attn_split_keys; /* 0: planner's choice; > 0: keys per split (rounded up to the
                              kernel's granule, 32 bf16 / 16 fp32)                        */
  int32_t linear_ksplit;   /* 0: planner's choice; > 0: reduction splits of st_linear (used
                              only when it divides K / 64)                                 */
  int32_t linear_stages;   /* 0 or 4: planner's choice (four-stage ring); 8: eight stages  */
  int32_t attn_balance;    /* 0: planner's choice; 1: one split size for the whole batch;
                              2: splits sized per request on the device (bf16, B <= 64)    */
  int32_t step_serial;     /* 0: planner's choice; 1: the verification step enqueues every
                              launch on the caller's stream (no side stream)              */
} st_testing_plan;

/* Installs `plan` for every later call in the process; NULL restores the
   planners' own choices.  Returns ST_OK, or ST_E_INVALID (nothing changed) for
   a field outside the ranges above.  Process-global and not thread-safe: set
   it, run the calls under test (workspace queries included: a size queried
   under one plan is valid only for calls under the same plan), reset it. */
int st_testing_set_plan(const st_testing_plan* plan);

#ifdef __cplusplus
}
#endif

#endif /* ST_TESTING_H */
