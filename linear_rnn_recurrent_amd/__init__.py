"""MI355X selective state update over a paged recurrent-state pool."""
