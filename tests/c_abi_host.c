/* The public header compiled as plain C99 and the library linked from C:
 * host-only calls (sizes, validation, error strings), no device needed. */
#include <stdio.h>
#include <string.h>

#include "dpo_head.h"

int main(void) {
  const size_t ws = dpo_workspace_bytes(DPO_OP_SEQ_LOGPS, 8, 2048, 4096, 128256);
  if (ws == 0) return 1;
  if (dpo_workspace_bytes(DPO_OP_SEQ_LOGPS, 3, 2048, 4096, 128256) != 0) return 2; /* odd rows */
  if (dpo_workspace_bytes(DPO_OP_HEAD_BACKWARD, 8, 2048, 100, 128256) != 0) return 3; /* H % 64 */
  /* validation happens before any launch: NULL pointers are refused */
  if (dpo_seq_logps(NULL, NULL, NULL, NULL, 8, 2048, 4096, 128256, NULL, NULL, NULL, NULL, NULL, ws, NULL) !=
      DPO_ERR_NULL)
    return 4;
  if (dpo_loss(NULL, NULL, 4, 0.1, DPO_PAIRS_ADJACENT, NULL, NULL, NULL, NULL, NULL, NULL) != DPO_ERR_NULL) return 5;
  const char* msg = dpo_strerror(DPO_ERR_SHAPE);
  if (!msg || strlen(msg) == 0) return 6;
  printf("c abi ok: workspace %zu bytes; %s\n", ws, msg);
  return 0;
}
